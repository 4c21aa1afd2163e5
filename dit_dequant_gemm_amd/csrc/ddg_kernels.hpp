// HIP kernels of libddg for gfx950 (CDNA4), templated on the bit width B.
//
//   quantize_pack_kernel  per-group(128) symmetric quantizer + MSB-first pack
//                         (Wan-Dancer-14B quantization report, §3.1, §3.3)
//   dequantize_kernel     dense bf16 w_hat (same report, §3.4)
//   gemm_large_kernel     Y = X w_hat^T for many tokens: bf16 MFMA, X tiles
//                         staged HBM->LDS, packed weights streamed to
//                         registers and dequantized there (§3.4 + §5.4)
//   gemm_small_kernel     the same product for M <= 64 tokens: a bandwidth
//                         kernel that streams the packed weights once
//   lowrank_t_kernel      T = bf16(X L1) for the low-rank branch (SVDQuant
//                         article, section "技术原理详解")
#pragma once

#include <type_traits>
#include <utility>

#include "ddg_device.hpp"

namespace ddg {

// ---------------------------------------------------------------------------
// K1: quantize + pack.  One lane per 32-weight chunk; the 4 lanes of a group
// are adjacent, so the group abs-max is a 2-step butterfly inside the quad.
// IEEE float32 throughout: correctly rounded multiply and divide (w / step by
// Markstein's correction, see div_markstein), round half to even, no other
// fused operations (the file is compiled with -ffp-contract=off), subnormals
// kept.
// ---------------------------------------------------------------------------
template <int B, bool F32_IN>
__global__ __launch_bounds__(256) void quantize_pack_kernel(const void* __restrict__ w,
                                                            int64_t n_chunks,
                                                            uint32_t* __restrict__ packed,
                                                            float* __restrict__ scales) {
  const int64_t c = (int64_t)blockIdx.x * 256 + threadIdx.x;
  const bool valid = c < n_chunks;
  float v[32];
  if (valid) {
    if constexpr (F32_IN) {
      const f32x4* src = reinterpret_cast<const f32x4*>(static_cast<const float*>(w) + c * 32);
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        const f32x4 t = src[i];
        v[4 * i] = t[0]; v[4 * i + 1] = t[1]; v[4 * i + 2] = t[2]; v[4 * i + 3] = t[3];
      }
    } else {
      const u32x4* src = reinterpret_cast<const u32x4*>(static_cast<const uint16_t*>(w) + c * 32);
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const u32x4 t = src[i];
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          v[8 * i + 2 * j] = bf16_bits_to_f32(t[j] & 0xFFFFu);
          v[8 * i + 2 * j + 1] = bf16_bits_to_f32(t[j] >> 16);
        }
      }
    }
  } else {
#pragma unroll
    for (int i = 0; i < 32; ++i) v[i] = 0.0f;
  }
  float a = 0.0f;
#pragma unroll
  for (int i = 0; i < 32; ++i) a = __builtin_fmaxf(a, __builtin_fabsf(v[i]));
  a = __builtin_fmaxf(a, __shfl_xor(a, 1));
  a = __builtin_fmaxf(a, __shfl_xor(a, 2));
  const float a1 = a * 1.01f;
  const float step = (2.0f * a1) / (float)((1 << B) - 1);
  const bool zero_group = !(step != 0.0f);
  constexpr float nh = (float)Bits<B>::n_half;
  const bool fast = markstein_ok(step);
  float r[32];
#pragma unroll
  for (int i = 0; i < 32; ++i) r[i] = v[i];
  quotients<32>(r, zero_group, fast, step, fast ? 1.0f / step : 0.0f);

  uint32_t out[B];
  uint64_t acc = 0;
  int nbits = 0, wo = 0;
#pragma unroll
  for (int i = 0; i < 32; ++i) {
    float q = __builtin_rintf(r[i]);
    q = __builtin_fminf(__builtin_fmaxf(q, -nh), nh);
    const uint32_t u = zero_group ? (uint32_t)Bits<B>::n_half
                                  : (uint32_t)((int)q + Bits<B>::n_half);
    acc = (acc << B) | u;
    nbits += B;
    if (nbits >= 32) {
      out[wo++] = __builtin_bswap32((uint32_t)(acc >> (nbits - 32)));
      nbits -= 32;
      acc &= (nbits ? ((1ull << nbits) - 1ull) : 0ull);
    }
  }
  if (valid) {
    uint32_t* dst = packed + c * B;
#pragma unroll
    for (int j = 0; j < B; ++j) dst[j] = out[j];
    if ((c & 3) == 0) scales[c >> 2] = step;
  }
}

// ---------------------------------------------------------------------------
// K5: dense dequantization, one lane per chunk (writes 32 bf16 = 64 bytes).
// ---------------------------------------------------------------------------
template <int B>
__global__ __launch_bounds__(256) void dequantize_kernel(const uint8_t* __restrict__ packed,
                                                         const float* __restrict__ scales,
                                                         int64_t n_chunks,
                                                         u32x4* __restrict__ out) {
  const int64_t c = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (c >= n_chunks) return;
  uint32_t raw[B], be[B];
  load_chunk<B>(packed + c * 4 * B, raw);
  byteswap_chunk<B>(raw, be);
  const float s = scales[c >> 2];
  const float ns64 = -64.0f * s;
  u32x4* dst = out + c * 4;
  dst[0] = __builtin_bit_cast(u32x4, dequant8<B>(raw, be, 0, s, ns64));
  dst[1] = __builtin_bit_cast(u32x4, dequant8<B>(raw, be, 1, s, ns64));
  dst[2] = __builtin_bit_cast(u32x4, dequant8<B>(raw, be, 2, s, ns64));
  dst[3] = __builtin_bit_cast(u32x4, dequant8<B>(raw, be, 3, s, ns64));
}

// ---------------------------------------------------------------------------
// Epilogue store of one 16x16 MFMA accumulator tile.  Lane (lr = lane%16,
// lq = lane/16) holds rows 4*lq .. 4*lq+3 of column lr.
// ---------------------------------------------------------------------------
template <bool OUT_BF16>
__device__ __forceinline__ void store_tile(void* __restrict__ y, int64_t ldy, int row0, int col,
                                           int m_rows, int n_cols, f32x4 v) {
  if (col >= n_cols) return;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int r = row0 + i;
    if (r < m_rows) {
      if constexpr (OUT_BF16) {
        static_cast<__bf16*>(y)[(int64_t)r * ldy + col] = (__bf16)v[i];
      } else {
        static_cast<float*>(y)[(int64_t)r * ldy + col] = v[i];
      }
    }
  }
}

// Low-rank term for one accumulator tile: acc += T[rows, :] * lora_up[cols, :]^T
// with T (M x R bf16) and lora_up (N x R bf16) read from global memory.
// Rows >= M of T read row M-1 (their outputs are never stored).
__device__ __forceinline__ bf16x8 load_bf16x8_or_zero(const __bf16* p, bool ok) {
  if (ok) return *reinterpret_cast<const bf16x8*>(p);
  return __builtin_bit_cast(bf16x8, u32x4{0u, 0u, 0u, 0u});
}

// ---------------------------------------------------------------------------
// K2: large-M GEMM.  Workgroup = 8 waves (512 threads, two per SIMD: one wave
// per SIMD cannot keep the matrix pipe busy), tile 256 rows x 256 columns.
// Wave w owns columns [32w, 32w + 32) for all 256 rows, so every packed
// weight is dequantized exactly once per workgroup and each wave needs only
// 128 accumulators.  MFMA v_mfma_f32_32x32x16_bf16: A = X rows (from LDS),
// B = dequantized weights (registers).
// K advances one 128-group per step of the outer loop:
//   * X[256 x 128] bf16 (64 KB) goes HBM -> LDS with buffer_load ... lds,
//     double-buffered (2 x 64 KB).  LDS row r holds 16 chunks of 16 bytes;
//     logical chunk c sits in slot c ^ (r & 15), which keeps the A-operand
//     ds_read_b128 free of bank conflicts.
//   * each lane streams its packed chunk (64 codes = 2B dwords) and scale one
//     group ahead into registers.
// The K index inside a group is permuted: MFMA k-step j (0..7), lane half h,
// element e uses input 64h + 8j + e, for the A operand and the dequantized B
// operand alike, so the dot products are unchanged.
// ---------------------------------------------------------------------------
struct GemmArgs {
  const __bf16* x;          // M x K
  const uint8_t* packed;    // N x K*B/8
  const float* scales;      // N x K/128
  void* y;                  // M x N
  const __bf16* t;          // M x R (low-rank intermediate) or null
  const __bf16* lora_up;    // N x R or null
  int m, n, k, r;
  int tiles_m, tiles_n;
  int out_bf16;             // 1: y is bf16, 0: y is float32
};

constexpr int kBM = 256;
constexpr int kBN = 256;
constexpr int kLdsStage = kBM * kGroup * 2;   // 64 KB

__device__ __forceinline__ void tile_coords(int bid, int tiles_m, int tiles_n, int& tm, int& tn) {
  // XCD-aware remap: consecutive workgroup ids go to the 8 XCDs round-robin;
  // give each XCD a contiguous range of tile ids so that the tiles sharing
  // X rows / weight columns share an L2.
  const int total = tiles_m * tiles_n;
  const int q = total / 8, rem = total % 8;
  const int xcd = bid % 8, idx = bid / 8;
  const int t = (xcd < rem) ? xcd * (q + 1) + idx : rem * (q + 1) + (xcd - rem) * q + idx;
  // grouped ordering inside the range: 4 tile rows share each column strip
  constexpr int GM = 4;
  const int group_size = GM * tiles_n;
  const int gid = t / group_size;
  const int first_m = gid * GM;
  const int gm = min(tiles_m - first_m, GM);
  const int in_group = t - gid * group_size;
  tm = first_m + in_group % gm;
  tn = in_group / gm;
}

__device__ __forceinline__ f32x16 mfma32x32x16(bf16x8 a, bf16x8 b, f32x16 c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}

// One 256 x 256 output tile (tile index `tile` of the product `args`); `lds`
// is the workgroup's 128 KB LDS block.  Kernels: gemm_large_kernel (one
// product) and gemm_grouped_large_kernel (several products in one launch).
template <int B>
__device__ __forceinline__ void large_tile(const GemmArgs& args, int tile, uint8_t* lds) {
  constexpr int RB = kBM / 32;          // 8 row blocks of 32
  constexpr int LA = 4;                 // A-operand look-ahead, in MFMA steps
  constexpr int RING = 8;               // A-operand ring (64 steps per group = 8 laps)
  constexpr int STEPS = 8 * RB;         // 8 k-steps x 8 row blocks
  constexpr int HAND = STEPS - LA;      // step of the group hand-over (barrier)
  constexpr int CW = 2 * B;             // packed dwords per lane per group
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int lane = threadIdx.x & 63;
  const int lr = lane & 31, lh = lane >> 5;
  int tm, tn;
  tile_coords(tile, args.tiles_m, args.tiles_n, tm, tn);
  const int m0 = tm * kBM;
  const int nw0 = tn * kBN;
  const int K = args.k;
  const int G = K / kGroup;
  const uint32_t row_bytes = (uint32_t)K * B / 8;
  const uint32_t xrow_bytes = (uint32_t)K * 2;
  const int m_valid = min(kBM, args.m - m0);
  const int n_valid = min(kBN, args.n - nw0);
  // Rows past M / columns past N read as zeros (their results are not stored).
  const rsrc_t rx = make_rsrc(args.x + (int64_t)m0 * K, (uint32_t)m_valid * xrow_bytes);
  const rsrc_t rw = make_rsrc(args.packed + (int64_t)nw0 * row_bytes, (uint32_t)n_valid * row_bytes);
  const rsrc_t rs = make_rsrc(args.scales + (int64_t)nw0 * G, (uint32_t)n_valid * G * 4);

  // X -> LDS.  DMA instruction i (0..7) of wave w fills 1 KB block 8w+i: rows
  // 32w + 4i + lane/16, slot lane%16, holding logical chunk slot ^ (row & 15).
  uint32_t xoff[4];
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const int r = wave * 32 + 4 * j + (lane >> 4);
    const int c = (lane & 15) ^ (r & 15);
    xoff[j] = (uint32_t)r * xrow_bytes + (uint32_t)c * 16;
  }
  auto issue_x_one = [&](int g, int stage, int i) {
    uint8_t* base = lds + stage * kLdsStage + wave * 8 * 1024;
    __builtin_amdgcn_raw_ptr_buffer_load_lds(rx, (lds_ptr_t)(base + i * 1024), 16,
                                             xoff[i & 3] + (uint32_t)(i >> 2) * 16 * xrow_bytes,
                                             (uint32_t)g * kGroup * 2, 0, 0);
  };

  // Packed chunk (codes 64h .. 64h+63 of column 32w + lane%32) and its scale.
  const uint32_t nl = (uint32_t)(wave * 32 + lr);
  const uint32_t woff = nl * row_bytes + (uint32_t)lh * 8 * B;
  const uint32_t soffs = nl * (uint32_t)G * 4;
  auto load_w = [&](int g, uint32_t (&w)[CW], float& sc) {
    load_chunk_buf<B>(rw, woff, (uint32_t)g * 16 * B, w);
    load_chunk_buf<B>(rw, woff + 4 * B, (uint32_t)g * 16 * B, w + B);
    sc = __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(rs, soffs,
                                                                      (uint32_t)g * 4, 0));
  };

  // A operand of step u (k-step u/8, row block u%8) from an LDS stage.
  uint32_t aoff[8];
#pragma unroll
  for (int ks = 0; ks < 8; ++ks) aoff[ks] = (uint32_t)(lr * 256 + (((8 * lh + ks) ^ (lr & 15)) * 16));
  auto read_a = [&](int stage, int u) -> bf16x8 {
    return *reinterpret_cast<const bf16x8*>(lds + stage * kLdsStage + (u & 7) * 8192 +
                                            aoff[u >> 3]);
  };

  f32x16 acc[RB];
#pragma unroll
  for (int rb = 0; rb < RB; ++rb)
#pragma unroll
    for (int i = 0; i < 16; ++i) acc[rb][i] = 0.f;

  if (args.t != nullptr) {
    // acc = T * lora_up^T over the rank dimension, 16 at a time (zero-padded).
    const int R = args.r;
    const bf16x8 zero = __builtin_bit_cast(bf16x8, u32x4{0u, 0u, 0u, 0u});
    const int n = min(nw0 + wave * 32 + lr, args.n - 1);
    for (int j0 = 0; j0 < R; j0 += 16) {
      const int kk = j0 + 8 * lh;
      const bool kok = kk < R;
      const int kc = min(kk, R - 8);
      const bf16x8 v = *reinterpret_cast<const bf16x8*>(args.lora_up + (int64_t)n * R + kc);
      const bf16x8 bl = kok ? v : zero;
#pragma unroll
      for (int rb = 0; rb < RB; ++rb) {
        const int m = min(m0 + rb * 32 + lr, args.m - 1);
        const bf16x8 tv = *reinterpret_cast<const bf16x8*>(args.t + (int64_t)m * R + kc);
        acc[rb] = mfma32x32x16(kok ? tv : zero, bl, acc[rb]);
      }
    }
  }

  uint32_t wc[CW], wn[CW], be[CW];
  float sc = 0.f, sn = 0.f, ns64 = 0.f;
  bf16x8 ring[RING];
  u32x4 bc, bnx;
  uint32_t nib[2];                      // 4-bit: spread nibbles of the current dword

  auto take_next_weights = [&]() {
#pragma unroll
    for (int j = 0; j < CW; ++j) wc[j] = wn[j];
    sc = sn;
    if constexpr (B != 4) {
#pragma unroll
      for (int j = 0; j < CW; ++j) be[j] = __builtin_bswap32(wc[j]);
    }
    ns64 = -64.0f * sc;
  };
  // dequantization job p (bf16 pair p, 0..3) of k-step ks
  auto dq_job = [&](int p, int ks) {
    if constexpr (B == 4) {
      if (p == 0) spread_nibbles(wc[ks], nib);
    }
    bnx[p] = dequant_pair<B>(be, nib, ks, p, sc, ns64);
  };

  // Group g uses LDS stage (g + G) % 2, so that after an optional lone first
  // group (odd G) the loop runs in (stage 0, stage 1) pairs.
  const int st0 = G & 1;
#pragma unroll
  for (int i = 0; i < 8; ++i) issue_x_one(0, st0, i);
  load_w(0, wn, sn);
  __builtin_amdgcn_s_waitcnt(0);
  __syncthreads();
  take_next_weights();
#pragma unroll
  for (int u = 0; u < LA; ++u) ring[u % RING] = read_a(st0, u);
#pragma unroll
  for (int p = 0; p < 4; ++p) dq_job(p, 0);
  bc = bnx;

  // One 128-group: 64 steps (8 k-steps x 8 row blocks), one MFMA each.  Every
  // step index is a compile-time constant (fold over an index sequence), so the
  // operand ring and the dequantization schedule are fully static:
  //   steps 0..7    one X DMA instruction each (next group -> idle stage)
  //   step 8        packed chunk + scale of the next group
  //   every step    one LDS read LA steps ahead; on even row blocks one
  //                 dequantization job (2 codes) for the next k-step; 1 MFMA
  //   end of ks = 6 switch to the next group's weights (their loads landed)
  //   step HAND     barrier: the next group's X is in LDS, this stage is free
  // The last group runs the same code: its "next group" is itself again
  // (clamped), fetched into the idle stage and never used.
  auto group = [&](int g, auto stage_tag) {
    constexpr int ST = decltype(stage_tag)::value;
    const int gn = min(g + 1, G - 1);
    auto step = [&]<int T>(std::integral_constant<int, T>) {
      constexpr int ks = T >> 3, rb = T & 7;
      if constexpr (T < 8) issue_x_one(gn, ST ^ 1, T);
      if constexpr (T == 8) load_w(gn, wn, sn);
      if constexpr (T == HAND) {
        __builtin_amdgcn_s_waitcnt(0);
        __syncthreads();
      }
      constexpr int u = T + LA;
      if constexpr (u < STEPS) {
        ring[u % RING] = read_a(ST, u);
      } else {
        ring[u % RING] = read_a(ST ^ 1, u - STEPS);
      }
      if constexpr ((rb & 1) == 0) dq_job(rb >> 1, (ks + 1) & 7);
      acc[rb] = mfma32x32x16(ring[T % RING], __builtin_bit_cast(bf16x8, bc), acc[rb]);
      if constexpr (rb == 7) {
        bc = bnx;
        if constexpr (ks == 6) take_next_weights();
      }
      // one MFMA, then the VALU work rides in its shadow
      __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
      __builtin_amdgcn_sched_group_barrier(0x002, 8, 0);
      __builtin_amdgcn_sched_barrier(0);
    };
    [&]<int... T>(std::integer_sequence<int, T...>) {
      (step(std::integral_constant<int, T>{}), ...);
    }(std::make_integer_sequence<int, STEPS>{});
  };

  using I0 = std::integral_constant<int, 0>;
  using I1 = std::integral_constant<int, 1>;
  int g = 0;
  if (st0 == 1) group(g++, I1{});
  for (; g < G; g += 2) {
    group(g, I0{});
    group(g + 1, I1{});
  }

  // Epilogue: every wave is done with LDS (the last group's reads run past
  // its barrier); each 32 x 32 block leaves through a 5 KB scratch per wave
  // as 16-byte pieces of rows.
  __syncthreads();
  float* scratch = reinterpret_cast<float*>(lds + wave * kEpiScratch);
  const bool vec = epi_vec_ok(args.y, args.n, args.out_bf16 != 0);
#pragma unroll
  for (int rb = 0; rb < RB; ++rb) {
    if (args.out_bf16)
      store_block32<true>(acc[rb], scratch, args.y, args.m, args.n, m0 + rb * 32, nw0 + wave * 32, vec);
    else
      store_block32<false>(acc[rb], scratch, args.y, args.m, args.n, m0 + rb * 32, nw0 + wave * 32, vec);
  }
}

template <int B>
__global__ __launch_bounds__(512, 1) void gemm_large_kernel(GemmArgs args) {
  __shared__ __attribute__((aligned(1024))) uint8_t lds[2 * kLdsStage];
  large_tile<B>(args, blockIdx.x, lds);
}

// ---------------------------------------------------------------------------
// K3: small-M GEMM (16 < M <= 64; M <= 16 when the skinny kernel below
// does not apply): a bandwidth kernel.
// Workgroup = NC x NK waves.  Wave (c, h) owns column block c (16 columns of
// the workgroup's 16*NC) and K split h (a contiguous range of 128-groups).
//   * X: for each group, the 16*RB x 128 bf16 slice of a K split is staged
//     into an LDS ring with coalesced buffer_load ... lds (1 KB per
//     instruction, shared out among the NC waves of that split) and read back
//     as MFMA A operands by all NC waves.  Rows past M read as zeros.
//   * packed weights: each lane's chunk (B dwords) and scale in a register
//     ring; the X slice and the weights of step j + D are issued together at
//     step j.
//   * the NK partial tiles of a column block are summed through LDS.
// Ring slots are static (the step loop is unrolled by the ring size).  In the
// main loop, group indices past a wave's range are clamped, loaded and never
// used; the last steps (the tail) issue nothing.
// ---------------------------------------------------------------------------
// LDS of the small-M kernel for a (RB, NC, NK) shape: the X ring (one array
// per slot, so that the compiler can see that a DMA into one slot does not
// alias reads of another, and does not make the reads wait for it) and the
// partial tiles of the K-split reduction.  A kernel declares it __shared__.
template <int RB, int NC, int NK>
struct SmallLds {
  static constexpr int XSLOT = RB * 16 * 256;        // one group's X slice: 16*RB rows x 256 bytes
  static constexpr int RED_BYTES = (NK > 1 ? NK - 1 : 1) * NC * RB * 64 * 16;
  // Ring slots: 3 with a two-way K split, else 2 (both within the 160 KB of
  // LDS).  Deeper rings measured slower on the 16- to 64-token products
  // (16 x 3072 x 3072: 5.1 us with 2 slots, 5.6 with 4): they hold more LDS
  // per workgroup, and near the end of a K range they fetch clamped groups
  // that are never used.
  static constexpr int S_FIT = (160 * 1024 - RED_BYTES) / (NK * XSLOT);
  static constexpr int S_WANT = NK <= 2 ? 3 : 2;
  static constexpr int S = S_FIT > S_WANT ? S_WANT : S_FIT;
  static_assert(S >= 2, "X ring needs two slots");
  __attribute__((aligned(1024))) uint8_t xs0[NK][XSLOT];
  __attribute__((aligned(1024))) uint8_t xs1[NK][XSLOT];
  __attribute__((aligned(1024))) uint8_t xs2[S > 2 ? NK : 1][S > 2 ? XSLOT : 16];
  __attribute__((aligned(1024))) uint8_t xs3[S > 3 ? NK : 1][S > 3 ? XSLOT : 16];
  __attribute__((aligned(1024))) uint8_t xs4[S > 4 ? NK : 1][S > 4 ? XSLOT : 16];
  __attribute__((aligned(1024))) uint8_t xs5[S > 5 ? NK : 1][S > 5 ? XSLOT : 16];
  f32x4 red[NK > 1 ? NK - 1 : 1][NC][RB][64];
};

// Workgroup `wg` of the product `args` (column block 16 NC wg ..).  Kernels:
// gemm_small_kernel (one product) and gemm_grouped_small_kernel (several).
template <int B, int RB, int NC, int NK>
__device__ __forceinline__ void small_body(const GemmArgs& args, int wg, SmallLds<RB, NC, NK>& L) {
  // X slices and packed weights of step j + D are issued together at step j
  // (ring of S = D + 1 slots each).  Loads finish in issue order, so waiting
  // for the X of step j never waits for a later step's packed weights.
  constexpr int XSLOT = SmallLds<RB, NC, NK>::XSLOT;
  constexpr int S = SmallLds<RB, NC, NK>::S;
  constexpr int D = S - 1;                    // steps in flight
  constexpr int DMA_SLOT = XSLOT / 1024;      // 1 KB DMA instructions per slice
  static_assert(DMA_SLOT % NC == 0, "slice DMA must split evenly over the column waves");
  constexpr int ND = DMA_SLOT / NC;           // DMA instructions per wave per group
  constexpr int NWL = (B == 3 || B == 4) ? 2 : 3;   // buffer loads per group: chunk + scale
  // issued after X(j) (at step j - D): W(j), then D - 1 steps of X + W
  constexpr int VM_AHEAD = NWL + (D - 1) * (ND + NWL);
  static_assert(VM_AHEAD < 64, "vmcnt field");

  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int c = wave % NC, h = wave / NC;
  auto xslot = [&]<int SL>(std::integral_constant<int, SL>) -> uint8_t* {
    if constexpr (SL == 0) return &L.xs0[h][0];
    else if constexpr (SL == 1) return &L.xs1[h][0];
    else if constexpr (SL == 2) return &L.xs2[h][0];
    else if constexpr (SL == 3) return &L.xs3[h][0];
    else if constexpr (SL == 4) return &L.xs4[h][0];
    else return &L.xs5[h][0];
  };
  const int lane = threadIdx.x & 63;
  const int lr = lane & 15, lq = lane >> 4;
  const int n0 = wg * 16 * NC;
  const int K = args.k;
  const int G = K / kGroup;
  const int g_begin = h * G / NK, g_end = (h + 1) * G / NK;
  const int cnt = g_end - g_begin;
  const int steps = (G + NK - 1) / NK;        // the same for every wave (barriers)
  const int g_last = cnt > 0 ? g_end - 1 : G - 1;
  const uint32_t row_bytes = (uint32_t)K * B / 8;

  // this wave's column (rows past N read as zeros through the resource bounds)
  const int n = min(n0 + c * 16 + lr, args.n - 1);
  const int n_valid = min(16 * NC, args.n - n0);
  const rsrc_t rw = make_rsrc(args.packed + (int64_t)n0 * row_bytes, (uint32_t)n_valid * row_bytes);
  const rsrc_t rs = make_rsrc(args.scales + (int64_t)n0 * G, (uint32_t)n_valid * G * 4);
  const uint32_t woff = (uint32_t)(c * 16 + lr) * row_bytes + (uint32_t)lq * 4 * B;
  const uint32_t soffs = (uint32_t)(c * 16 + lr) * (uint32_t)G * 4;

  // X DMA: instruction d of this wave fills 1 KB block c*ND + d of the slice:
  // rows 4*(c*ND+d) + lane/16, slot lane%16 = logical chunk ^ (row & 15).
  const rsrc_t rx = make_rsrc(args.x, (uint32_t)args.m * (uint32_t)K * 2);
  auto issue_x = [&](uint8_t* slot_base, int j) {
    const int g = min(g_begin + j, g_last);
    uint8_t* base = slot_base + (c * ND) * 1024;
#pragma unroll
    for (int d = 0; d < ND; ++d) {
      const int row = 4 * (c * ND + d) + (lane >> 4);
      const uint32_t voff = (uint32_t)row * (uint32_t)K * 2 + (uint32_t)(((lane & 15) ^ (row & 15)) * 16);
      __builtin_amdgcn_raw_ptr_buffer_load_lds(rx, (lds_ptr_t)(base + d * 1024), 16, voff,
                                               (uint32_t)g * kGroup * 2, 0, 0);
    }
  };
  uint32_t aoff[4];
#pragma unroll
  for (int s = 0; s < 4; ++s) aoff[s] = (uint32_t)(lr * 256 + (((4 * lq + s) ^ lr) * 16));

  uint32_t raw[S][B];
  float sc[S];
  auto load_w = [&](int slot, int j) {
    const int g = min(g_begin + j, g_last);
    load_chunk_buf<B>(rw, woff, (uint32_t)g * 16 * B, raw[slot]);
    sc[slot] = __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(rs, soffs,
                                                                            (uint32_t)g * 4, 0));
  };

  // one accumulator per sub-step: the four MFMAs of a group are independent
  // (a single chain would wait out the MFMA latency four times per group)
  f32x4 acc4[4][RB];
#pragma unroll
  for (int s = 0; s < 4; ++s)
#pragma unroll
    for (int rb = 0; rb < RB; ++rb) acc4[s][rb] = f32x4{0.f, 0.f, 0.f, 0.f};

  auto compute = [&](const uint8_t* base, int ws) {
    // plus-one dequantization (see dequant8_p1)
    uint32_t be1[B];
    if constexpr (B != 4) plus_one_words<B>(raw[ws], be1);
    const float nsh = -(float)(1 << (B - 1)) * sc[ws];
#pragma unroll
    for (int s = 0; s < 4; ++s) {
      const uint32_t x1 = B == 4 ? raw[ws][s] + 0x11111111u : 0u;
      const bf16x8 bf = dequant8_p1<B>(be1, x1, s, sc[ws], nsh);
#pragma unroll
      for (int rb = 0; rb < RB; ++rb) {
        const bf16x8 a = *reinterpret_cast<const bf16x8*>(base + rb * 4096 + aoff[s]);
        acc4[s][rb] = mfma16x16x32(a, bf, acc4[s][rb]);
      }
    }
  };

  // Step j (ring slot j % S for both rings): wait for X(j), barrier, issue
  // X(j+D) and W(j+D) into slot (j-1) % S, compute step j.
  //
  // The wait leaves in flight exactly the loads issued after X(j): W(j), then
  // X and W of every later step issued so far.  In the main loop that is D - 1
  // steps; at tail step U (which issues nothing: its loads would be for steps
  // past the end) it is D - 1 - U.  The count must be exact, not an upper
  // bound: with fewer loads in flight than it allows, the wait would pass with
  // this wave's share of X(j) still landing, and the barrier would hand the
  // slot to the other column waves too early.  (A tail that issued loads would
  // break it: their registers are never read, so the compiler drops the weight
  // loads and keeps only the DMAs.)
  using std::integral_constant;
  constexpr auto vm_imm = [](int v) { return (v & 15) | ((v >> 4) << 14) | (7 << 4) | (15 << 8); };
  auto step = [&]<int U, bool TAIL>(integral_constant<int, U>, std::bool_constant<TAIL>, int j) {
    // own X DMA of step j landed; then every wave's has, and every wave is
    // done with slot (j-1) % S.  A bare s_barrier: a fenced barrier would
    // also wait for the loads of later steps still in flight.
    constexpr int AHEAD = TAIL ? NWL + (D - 1 - U) * (ND + NWL) : VM_AHEAD;
    static_assert(AHEAD >= NWL && AHEAD < 64, "vmcnt field");
    __builtin_amdgcn_s_waitcnt(vm_imm(AHEAD));
    asm volatile("s_barrier" ::: "memory");
    if constexpr (!TAIL) {
      issue_x(xslot(integral_constant<int, (U + D) % S>{}), j + D);
      __builtin_amdgcn_sched_barrier(0);
      load_w((U + D) % S, j + D);
      __builtin_amdgcn_sched_barrier(0);
    }
    if (j < cnt) compute(xslot(integral_constant<int, U % S>{}), U % S);
  };
  // prologue: steps 0..D-1, X then W per step (the order of the steady state)
  [&]<int... J>(std::integer_sequence<int, J...>) {
    // (sched_barrier on both sides of the weight loads: the scheduler would
    // otherwise move them among or ahead of the X DMAs, or sink the scale
    // loads to the end, and the counted waits above assume this order)
    ((issue_x(xslot(integral_constant<int, J>{}), J), __builtin_amdgcn_sched_barrier(0),
      load_w(J, J), __builtin_amdgcn_sched_barrier(0)), ...);
  }(std::make_integer_sequence<int, D>{});
  // main loop: whole blocks of S steps, every load unconditional (so the
  // compiler's wait counts stay exact across the loop, and no load is dead)
  const int full = steps / S * S;
  for (int j0 = 0; j0 < full; j0 += S) {
    [&]<int... U>(std::integer_sequence<int, U...>) {
      (step(integral_constant<int, U>{}, std::false_type{}, j0 + U), ...);
    }(std::make_integer_sequence<int, S>{});
  }
  // tail: the remaining steps (at most S - 1 = D)
  [&]<int... U>(std::integer_sequence<int, U...>) {
    ([&] { if (full + U < steps) step(integral_constant<int, U>{}, std::true_type{}, full + U); }(), ...);
  }(std::make_integer_sequence<int, S - 1>{});
  __syncthreads();

  f32x4 acc[RB];
#pragma unroll
  for (int rb = 0; rb < RB; ++rb)
#pragma unroll
    for (int i = 0; i < 4; ++i)
      acc[rb][i] = (acc4[0][rb][i] + acc4[1][rb][i]) + (acc4[2][rb][i] + acc4[3][rb][i]);

  if constexpr (NK > 1) {
    if (h > 0) {
#pragma unroll
      for (int rb = 0; rb < RB; ++rb) L.red[h - 1][c][rb][lane] = acc[rb];
    }
    __syncthreads();
    if (h > 0) return;
#pragma unroll
    for (int k = 0; k < NK - 1; ++k)
#pragma unroll
      for (int rb = 0; rb < RB; ++rb) {
        const f32x4 v = L.red[k][c][rb][lane];
        acc[rb][0] += v[0]; acc[rb][1] += v[1]; acc[rb][2] += v[2]; acc[rb][3] += v[3];
      }
  }

  if (args.t != nullptr) {
    const int R_ = args.r;
    const bf16x8 zero = __builtin_bit_cast(bf16x8, u32x4{0u, 0u, 0u, 0u});
    for (int j0 = 0; j0 < R_; j0 += 32) {
      const int kk = j0 + 8 * lq;
      const bool kok = kk < R_;
      const int kc = min(kk, R_ - 8);
      const bf16x8 vl = *reinterpret_cast<const bf16x8*>(args.lora_up + (int64_t)n * R_ + kc);
      const bf16x8 bl = kok ? vl : zero;
#pragma unroll
      for (int rb = 0; rb < RB; ++rb) {
        const int m = min(rb * 16 + lr, args.m - 1);
        const bf16x8 vt = *reinterpret_cast<const bf16x8*>(args.t + (int64_t)m * R_ + kc);
        acc[rb] = mfma16x16x32(kok ? vt : zero, bl, acc[rb]);
      }
    }
  }

#pragma unroll
  for (int rb = 0; rb < RB; ++rb) {
    if (args.out_bf16)
      store_tile<true>(args.y, args.n, rb * 16 + 4 * lq, n0 + c * 16 + lr, args.m, args.n, acc[rb]);
    else
      store_tile<false>(args.y, args.n, rb * 16 + 4 * lq, n0 + c * 16 + lr, args.m, args.n, acc[rb]);
  }
}

template <int B, int RB, int NC, int NK>
__global__ __launch_bounds__(64 * NC * NK) void gemm_small_kernel(GemmArgs args) {
  __shared__ SmallLds<RB, NC, NK> L;
  small_body<B, RB, NC, NK>(args, blockIdx.x, L);
}

// ---------------------------------------------------------------------------
// K3s: product for M <= 16 tokens that streams the packed weights.
// Workgroup = 8 waves = an 8-way split of the K groups; it owns NCB blocks of
// 16 output columns.  Wave h works through its share of K in chunks of
// kc <= KC groups: the chunk's X slice is loaded once into registers and run
// against the packed rows of every column block, so the weights are read
// once and X once per workgroup.
//   * scales: the workgroup's rows of the scale matrix are one contiguous
//     range; it is copied to LDS once (dynamic LDS, 16 NCB G floats).
//   * packed weights of a (column block, chunk) -- 16 rows x kc*16*B bytes,
//     each row's part contiguous -- go to the wave's own LDS buffer with 1 KB
//     buffer_load ... lds instructions whose lanes take consecutive 16-byte
//     pieces (whole cache lines, rows end to end); lane (lr, lq) then reads
//     its B dwords per group: inputs 32 lq .. 32 lq + 31 of the group, the
//     input order of the other kernels (the X operand uses it too).
//   * dequantization in the plus-one form (see dequant8_p1).
// The next column block (or block 0 of the next chunk) streams into the other
// buffer while this one is dequantized and multiplied.  A load with nothing
// to fetch goes to an offset past the end of its buffer resource (in the
// offset register: that is what the range check sees) and returns zeros
// without a memory access.
// ---------------------------------------------------------------------------
// LDS bytes of gemm_skinny_kernel<B, KC, NCB>: the weight buffers (the first
// one also holds the final reduction) plus the per-wave scale areas.
__host__ __device__ constexpr size_t skinny_static_lds(int b, int kc, int ncb) {
  return (size_t)8 * ((kc * b + 3) / 4) * 1024 * 2 >= (size_t)8 * ((kc * b + 3) / 4) * 1024 + (size_t)8 * ncb * 1024
             ? (size_t)8 * ((kc * b + 3) / 4) * 1024 * 2
             : (size_t)8 * ((kc * b + 3) / 4) * 1024 + (size_t)8 * ncb * 1024;
}
__host__ __device__ constexpr size_t skinny_scale_lds(int kc) { return (size_t)8 * kc * 64 * 4; }
constexpr size_t kLdsLimit = 160 * 1024;

// LDS layout of the skinny kernel body: two weight buffers (separate arrays,
// so that the compiler can tell that a DMA into one does not feed reads of
// the other, and does not wait for it; the first also holds the final
// reduction) and the per-wave scale areas [wave][group j][row].
template <int B, int KC, int NCB>
struct SkinnyLds {
  static constexpr int NW = 8;
  static constexpr int NDMA = (KC * B + 3) / 4;       // 1 KB DMA instructions per wave per block
  static constexpr int WBUF = NDMA * 1024;
  static constexpr int RED = NW * NCB * 64 * 16;
  static constexpr int W0 = NW * WBUF >= RED ? NW * WBUF : RED;
  static constexpr int W1 = NW * WBUF;
};

// Workgroup wg of the product `args` (see the comment above).  wl0, wl1 and
// scw are LDS arrays of at least SkinnyLds<B, KC, NCB>::W0, ::W1 bytes and
// [8][KC][64] floats.
template <int B, int KC, int NCB>
__device__ __forceinline__ void skinny_body(const GemmArgs& args, int wg, uint8_t* wl0, uint8_t* wl1,
                                            float (*scw)[KC][64]) {
  constexpr int NW = SkinnyLds<B, KC, NCB>::NW;       // waves = K splits
  constexpr uint32_t kNoLoad = 0x80000000u;
  constexpr int NDMA = SkinnyLds<B, KC, NCB>::NDMA;
  constexpr int WBUF = SkinnyLds<B, KC, NCB>::WBUF;

  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int lane = threadIdx.x & 63;
  const int lr = lane & 15, lq = lane >> 4;
  const int K = args.k, G = K / kGroup;
  const int n0 = wg * 16 * NCB;
  // (wave-uniform: kept in scalar registers)
  const int gs = __builtin_amdgcn_readfirstlane(wave * G / NW);
  const int cnt = __builtin_amdgcn_readfirstlane((wave + 1) * G / NW) - gs;
  const int nch = __builtin_amdgcn_readfirstlane((cnt + KC - 1) / KC);
  const int kc_lo = __builtin_amdgcn_readfirstlane(cnt / max(nch, 1));
  const int kc_rem = cnt - kc_lo * nch;
  const uint32_t row_bytes = (uint32_t)K * B / 8;
  const int n_valid = min(16 * NCB, args.n - n0);
  const rsrc_t rw = make_rsrc(args.packed + (int64_t)n0 * row_bytes, (uint32_t)n_valid * row_bytes);
  const rsrc_t rs = make_rsrc(args.scales + (int64_t)n0 * G, (uint32_t)n_valid * G * 4);
  const rsrc_t rx = make_rsrc(args.x, (uint32_t)args.m * (uint32_t)K * 2);

  // chunk c of this wave: groups [g0, g0 + kc), balanced, kc <= KC
  auto chunk_g0 = [&](int c) __attribute__((always_inline)) { return gs + c * kc_lo + min(c, kc_rem); };
  auto chunk_kc = [&](int c) __attribute__((always_inline)) { return kc_lo + (c < kc_rem ? 1 : 0); };

  // Per-chunk DMA offsets: DMA d, lane i fetches piece f = 64 d + i of the
  // block (row f / (kc B), 16-byte piece f % (kc B) of that row's part);
  // pieces past the block, and every piece of a chunk past the last, get the
  // no-load offset.  f / (kc B) = f * inv >> 16 for f < 64 NDMA <= 576.
  auto chunk_offsets = [&](int c, uint32_t* off) __attribute__((always_inline)) {
    const bool valid = c < nch;
    const int g0 = chunk_g0(c), kc = chunk_kc(c);
    const uint32_t per_row = (uint32_t)(kc * B);
    const uint32_t inv = (65536u + per_row - 1) / per_row;
#pragma unroll
    for (int d = 0; d < NDMA; ++d) {
      const uint32_t f = 64 * d + lane;
      const uint32_t row = __umul24(f, inv) >> 16;
      const uint32_t piece = f - __umul24(row, per_row);
      off[d] = valid && f < 16u * per_row
                   ? __umul24(row, row_bytes) + (uint32_t)g0 * 16 * B + piece * 16
                   : kNoLoad;
    }
  };
  auto load_w = [&]<int BUF>(std::integral_constant<int, BUF>, int cb, const uint32_t* off)
      __attribute__((always_inline)) {
    uint8_t* dst = (BUF == 0 ? wl0 : wl1) + wave * WBUF;
    const uint32_t blk = (uint32_t)(cb * 16) * row_bytes;
#pragma unroll
    for (int d = 0; d < NDMA; ++d)
      __builtin_amdgcn_raw_ptr_buffer_load_lds(rw, (lds_ptr_t)(dst + d * 1024), 16, off[d] + blk, 0, 0, 0);
  };

  // scales of chunk c for the workgroup's rows -> scw[wave]: one 256-byte
  // DMA per group, lane i = row i (4 bytes per lane: no load straddles the
  // end of the resource)
  auto load_scales = [&](int c) __attribute__((always_inline)) {
    const int g0 = chunk_g0(c), kc = chunk_kc(c);
#pragma unroll
    for (int j = 0; j < KC; ++j) {
      const bool ok = c < nch && j < kc && lane < 16 * NCB;
      __builtin_amdgcn_raw_ptr_buffer_load_lds(rs, (lds_ptr_t)&scw[wave][j][0], 4,
                                               ok ? ((uint32_t)lane * G + g0 + j) * 4 : kNoLoad, 0, 0, 0);
    }
  };

  bf16x8 xa[KC][4];
  auto load_x = [&](int c) __attribute__((always_inline)) {
    const int g0 = chunk_g0(c), kc = chunk_kc(c);
    const uint32_t base = (uint32_t)lr * K * 2 + (uint32_t)(g0 * kGroup + 32 * lq) * 2;
#pragma unroll
    for (int j = 0; j < KC; ++j) {
      const bool ok = c < nch && j < kc;
#pragma unroll
      for (int t = 0; t < 4; ++t)
        xa[j][t] = __builtin_bit_cast(
            bf16x8, __builtin_amdgcn_raw_buffer_load_b128(rx, ok ? base + (j * kGroup + 8 * t) * 2 : kNoLoad, 0, 0));
    }
  };

  f32x4 acc[NCB][2];
#pragma unroll
  for (int cb = 0; cb < NCB; ++cb) acc[cb][0] = acc[cb][1] = f32x4{0.f, 0.f, 0.f, 0.f};

  // groups j >= kc (a short chunk) have zero X, so they add exact zeros
  auto compute = [&]<int BUF>(std::integral_constant<int, BUF>, int cb, int c) __attribute__((always_inline)) {
    const int kc = chunk_kc(c);
    const uint8_t* src = (BUF == 0 ? wl0 : wl1) + wave * WBUF + lr * (kc * B * 16) + lq * 4 * B;
#pragma unroll
    for (int j = 0; j < KC; ++j) {
      uint32_t r[B];
#pragma unroll
      for (int e = 0; e < B; ++e) r[e] = reinterpret_cast<const uint32_t*>(src + j * 16 * B)[e];
      const float s = scw[wave][min(j, kc - 1)][cb * 16 + lr];
      const float nsh = -(float)(1 << (B - 1)) * s;
      uint32_t be1[B];
      if constexpr (B != 4) plus_one_words<B>(r, be1);
#pragma unroll
      for (int t = 0; t < 4; ++t) {
        const uint32_t x1 = B == 4 ? r[t] + 0x11111111u : 0u;
        acc[cb][t & 1] = mfma16x16x32(xa[j][t], dequant8_p1<B>(be1, x1, t, s, nsh), acc[cb][t & 1]);
      }
    }
  };

  // Block (c, cb) uses weight buffer (c * NCB + cb) & 1; with NCB odd the
  // chunk loop is unrolled by two so that every buffer index is static.
  constexpr int CU = (NCB & 1) ? 2 : 1;
  using std::integral_constant;
  uint32_t off_cur[NDMA], off_next[NDMA];
  chunk_offsets(0, off_cur);
  load_w(integral_constant<int, 0>{}, 0, off_cur);
  auto block = [&]<int U, int CB>(integral_constant<int, U>, integral_constant<int, CB>, int c)
      __attribute__((always_inline)) {
    constexpr int cur = (U * NCB + CB) & 1;
    if constexpr (CB + 1 < NCB) {
      load_w(integral_constant<int, cur ^ 1>{}, CB + 1, off_cur);
    } else {
      chunk_offsets(c + 1, off_next);
      load_w(integral_constant<int, cur ^ 1>{}, 0, off_next);
    }
    // the scheduler would otherwise mix blocks (and their register reuse)
    __builtin_amdgcn_sched_barrier(0);
    if (c < nch) compute(integral_constant<int, cur>{}, CB, c);
    __builtin_amdgcn_sched_barrier(0);
  };
  auto chunk_body = [&]<int U>(integral_constant<int, U> u, int c) __attribute__((always_inline)) {
    load_scales(c);
    load_x(c);
    __builtin_amdgcn_sched_barrier(0);
    [&]<int... CB>(std::integer_sequence<int, CB...>) __attribute__((always_inline)) {
      (block(u, integral_constant<int, CB>{}, c), ...);
    }(std::make_integer_sequence<int, NCB>{});
#pragma unroll
    for (int d = 0; d < NDMA; ++d) off_cur[d] = off_next[d];
  };
  for (int c0 = 0; c0 < nch; c0 += CU) {
    [&]<int... U>(std::integer_sequence<int, U...>) __attribute__((always_inline)) {
      (chunk_body(integral_constant<int, U>{}, c0 + U), ...);
    }(std::make_integer_sequence<int, CU>{});
  }

  // sum the 8 partial tiles of each column block; wave cb finishes block cb
  // (the reduction reuses the first weight buffer: every DMA must have landed)
  __builtin_amdgcn_s_waitcnt(0);
  __syncthreads();
  f32x4* red = reinterpret_cast<f32x4*>(wl0);     // [NW][NCB][64]
#pragma unroll
  for (int cb = 0; cb < NCB; ++cb) {
    f32x4 v = acc[cb][0];
    v[0] += acc[cb][1][0]; v[1] += acc[cb][1][1]; v[2] += acc[cb][1][2]; v[3] += acc[cb][1][3];
    red[(wave * NCB + cb) * 64 + lane] = v;
  }
  __syncthreads();
  if (wave >= NCB) return;
  const int cb = wave;
  f32x4 tot = red[cb * 64 + lane];
#pragma unroll
  for (int w = 1; w < NW; ++w) {
    const f32x4 v = red[(w * NCB + cb) * 64 + lane];
    tot[0] += v[0]; tot[1] += v[1]; tot[2] += v[2]; tot[3] += v[3];
  }
  const int n = min(n0 + cb * 16 + lr, args.n - 1);
  if (args.t != nullptr) {
    const int R_ = args.r;
    const bf16x8 zero = __builtin_bit_cast(bf16x8, u32x4{0u, 0u, 0u, 0u});
    for (int j0 = 0; j0 < R_; j0 += 32) {
      const int kk = j0 + 8 * lq;
      const bool kok = kk < R_;
      const int kc = min(kk, R_ - 8);
      const bf16x8 bl = kok ? *reinterpret_cast<const bf16x8*>(args.lora_up + (int64_t)n * R_ + kc) : zero;
      const int m = min(lr, args.m - 1);
      const bf16x8 vt = *reinterpret_cast<const bf16x8*>(args.t + (int64_t)m * R_ + kc);
      tot = mfma16x16x32(kok ? vt : zero, bl, tot);
    }
  }
  if (args.out_bf16)
    store_tile<true>(args.y, args.n, 4 * lq, n0 + cb * 16 + lr, args.m, args.n, tot);
  else
    store_tile<false>(args.y, args.n, 4 * lq, n0 + cb * 16 + lr, args.m, args.n, tot);
}

template <int B, int KC, int NCB>
__global__ __launch_bounds__(512) void gemm_skinny_kernel(GemmArgs args) {
  using L = SkinnyLds<B, KC, NCB>;
  __shared__ __attribute__((aligned(1024))) uint8_t wl0[L::W0];
  __shared__ __attribute__((aligned(1024))) uint8_t wl1[L::W1];
  __shared__ __attribute__((aligned(256))) float scw[L::NW][KC][64];
  skinny_body<B, KC, NCB>(args, blockIdx.x, wl0, wl1, scw);
}

// ---------------------------------------------------------------------------
// K3g: several independent products with M <= 16 (mixed bit widths) in one
// launch -- e.g. the q, k and v projections of a block quantized to
// different widths, which cannot share one packed tensor.  Workgroup i runs
// workgroup i - wg_start[j] of product j (wg_start is a prefix sum over the
// products' workgroup counts); the body is the K3s one, chosen per product
// by bit width and chunk size.  The LDS arrays are sized for the widest case.
// ---------------------------------------------------------------------------
constexpr int kMaxGroup = 16;
constexpr int kGroupedNcb = 4;

struct GroupArgs {
  GemmArgs g[kMaxGroup];
  int wg_start[kMaxGroup + 1];
  int bits[kMaxGroup];
  int kc[kMaxGroup];
  int count;
};

// Up to kMaxGroup products with M > 64 in one launch of K2 tiles:
// tile_start is the prefix sum of the products' tile counts (tiles_m x
// tiles_n of each GemmArgs).
struct GroupLargeArgs {
  GemmArgs g[kMaxGroup];
  int tile_start[kMaxGroup + 1];
  int bits[kMaxGroup];
  int count;
};

// gemm_grouped_skinny_kernel(GroupArgs) and gemm_grouped_large_kernel
// (GroupLargeArgs) are defined in grouped.hip.

// ---------------------------------------------------------------------------
// K4: T = bf16(X * L1), with L1^T = lora_down (R x K) -- computed as
// T^T = lora_down * X^T so both MFMA operands are contiguous 16-byte reads.
// Workgroup = 4 waves over 16 token rows; waves split K in 32-wide steps;
// the 4 partials are summed through LDS, then rounded to bf16 once.
// ---------------------------------------------------------------------------
template <int RBLK>
__global__ __launch_bounds__(256) void lowrank_t_kernel(const __bf16* __restrict__ x,
                                                        const __bf16* __restrict__ lora_down,
                                                        __bf16* __restrict__ t, int m, int k,
                                                        int r) {
  __shared__ f32x4 red[4][RBLK][64];
  const int wave = threadIdx.x >> 6;
  const int lane = threadIdx.x & 63;
  const int lr = lane & 15, lq = lane >> 4;
  const int m0 = blockIdx.x * 16;
  const int mrow = min(m0 + lr, m - 1);
  const __bf16* xrow = x + (int64_t)mrow * k + 8 * lq;
  f32x4 acc[RBLK];
#pragma unroll
  for (int j = 0; j < RBLK; ++j) acc[j] = f32x4{0.f, 0.f, 0.f, 0.f};
  for (int k0 = wave * 32; k0 < k; k0 += 128) {
    const bf16x8 b = *reinterpret_cast<const bf16x8*>(xrow + k0);
#pragma unroll
    for (int j = 0; j < RBLK; ++j) {
      const int rr = j * 16 + lr;
      const bf16x8 a = load_bf16x8_or_zero(lora_down + (int64_t)min(rr, r - 1) * k + k0 + 8 * lq,
                                           rr < r);
      acc[j] = mfma16x16x32(a, b, acc[j]);
    }
  }
#pragma unroll
  for (int j = 0; j < RBLK; ++j) red[wave][j][lane] = acc[j];
  __syncthreads();
  if (wave == 0) {
    const int mm = m0 + lr;
#pragma unroll
    for (int j = 0; j < RBLK; ++j) {
      f32x4 s = red[0][j][lane];
#pragma unroll
      for (int w = 1; w < 4; ++w) {
        const f32x4 v = red[w][j][lane];
        s[0] += v[0]; s[1] += v[1]; s[2] += v[2]; s[3] += v[3];
      }
      const int rr = j * 16 + 4 * lq;      // rows rr..rr+3 of T^T = columns of T
      if (mm < m && rr < r) {
        // r % 8 == 0 and rr % 4 == 0, so rr < r implies rr + 3 < r
        uint32_t lo = pack_bf16x2(s[0], s[1]);
        uint32_t hi = pack_bf16x2(s[2], s[3]);
        u32x2 v = {lo, hi};
        *reinterpret_cast<u32x2*>(t + (int64_t)mm * r + rr) = v;
      }
    }
  }
}

}  // namespace ddg
