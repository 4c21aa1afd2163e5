// HIP kernels of libddg for gfx950 (CDNA4), templated on the bit width B.
//
//   quantize_pack_kernel  per-group(128) symmetric quantizer + MSB-first pack
//                         (Wan-Dancer-14B quantization report, §3.1, §3.3)
//   dequantize_kernel     dense bf16 w_hat (same report, §3.4)
//   gemm_large_kernel     Y = X w_hat^T for many tokens: bf16 MFMA, X tiles
//                         staged HBM->LDS, packed weights streamed to
//                         registers and dequantized there (§3.4 + §5.4)
//   gemm_n192_kernel      the same with 256 x 192 tiles, for outputs that
//                         256 x 256 tiles cover with compute units left idle
//   gemm_streamk_kernel   the same with K split across workgroups (split-K,
//                         stream-K) for products with few tiles
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
// lq = lane/16) holds rows 4*lq .. 4*lq+3 of column lr; row0 = 16 rb + 4 lq
// and col = 16 cb + lr for a tile (rb, cb) that is the same for all lanes.
// ---------------------------------------------------------------------------
template <bool OUT_BF16>
__device__ __forceinline__ void store_tile(void* __restrict__ y, int64_t ldy, int row0, int col,
                                           int m_rows, int n_cols, f32x4 v) {
  // a 16 x 16 tile wholly inside Y: no per-lane checks (one uniform branch;
  // 16 x 3072 x 3072: 6.29 -> 6.17 us, 16 x 640 x 5120: 7.68 -> 6.29 us)
  if (__builtin_amdgcn_readfirstlane(row0 & ~15) + 16 <= m_rows &&
      __builtin_amdgcn_readfirstlane(col & ~15) + 16 <= n_cols) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      if constexpr (OUT_BF16)
        static_cast<__bf16*>(y)[(int64_t)(row0 + i) * ldy + col] = (__bf16)v[i];
      else
        static_cast<float*>(y)[(int64_t)(row0 + i) * ldy + col] = v[i];
    }
    return;
  }
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

// 8 bf16 at p, or zeros where ok is false.  p must be a valid address even
// where ok is false (callers clamp the row):
// the load always runs and the select zeroes the lanes past the end.  (A
// branch around the load, which the lanes take differently, made the
// low-rank pre-pass about 7% slower in the fused 4096 x 3072 x 3072 call.)
__device__ __forceinline__ bf16x8 load_bf16x8_or_zero(const __bf16* p, bool ok) {
  const u32x4 v = *reinterpret_cast<const u32x4*>(p);
  return __builtin_bit_cast(bf16x8, ok ? v : u32x4{0u, 0u, 0u, 0u});
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

template <int GM = 4>
__device__ __forceinline__ void tile_coords(int bid, int tiles_m, int tiles_n, int& tm, int& tn) {
  // XCD-aware remap: consecutive workgroup ids go to the 8 XCDs round-robin;
  // give each XCD a contiguous range of tile ids so that the tiles sharing
  // X rows / weight columns share an L2.
  const int total = tiles_m * tiles_n;
  const int q = total / 8, rem = total % 8;
  const int xcd = bid % 8, idx = bid / 8;
  const int t = (xcd < rem) ? xcd * (q + 1) + idx : rem * (q + 1) + (xcd - rem) * q + idx;
  // grouped ordering inside the range: GM tile rows share each column strip
  const int group_size = GM * tiles_n;
  const int gid = t / group_size;
  const int first_m = gid * GM;
  const int gm = min(tiles_m - first_m, GM);
  const int in_group = t - gid * group_size;
  tm = first_m + in_group % gm;
  tn = in_group / gm;
}

// Tile t of the stream-K order: tiles in groups of 4 tile rows per column
// strip (the ranges of an XCD then cover few X row strips and few weight
// column strips).
__device__ __forceinline__ void tile_coords_range(int t, int tiles_m, int tiles_n, int& tm, int& tn) {
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

// Groups [g0, g1) of the 256 x 256 output tile (tm, tn) of the product
// `args`, added into acc (8 row blocks of the 32x32 accumulator layout; wave w
// holds columns 32w..32w+31).  With `lowrank` set, the branch term
// T * lora_up^T of the tile is added first.  `lds` is the workgroup's 128 KB
// LDS block; on return the last group's LDS reads may still be pending in
// other waves (a barrier must precede any reuse of LDS).
template <int B>
__device__ __forceinline__ void large_accumulate(const GemmArgs& args, int tm, int tn, int g0, int g1,
                                                 bool lowrank, f32x16 (&acc)[kBM / 32], uint8_t* lds) {
  constexpr int RB = kBM / 32;          // 8 row blocks of 32
  constexpr int LA = 4;                 // A-operand look-ahead, in MFMA steps
  constexpr int RING = 8;               // A-operand ring (64 steps per group = 8 laps)
  constexpr int STEPS = 8 * RB;         // 8 k-steps x 8 row blocks
  constexpr int HAND = STEPS - LA;      // step of the group hand-over (barrier)
  constexpr int CW = 2 * B;             // packed dwords per lane per group
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int lane = threadIdx.x & 63;
  const int lr = lane & 31, lh = lane >> 5;
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
    ns64 = (B == 4 ? -8.0f : -64.0f) * sc;   // dequant_pair's offset
  };
  // dequantization job p (bf16 pair p, 0..3) of k-step ks
  auto dq_job = [&](int p, int ks) {
    if constexpr (B == 4) {
      if (p == 0) spread_nibbles(wc[ks], nib);
    }
    bnx[p] = dequant_pair<B>(be, nib, ks, p, sc, ns64);
  };

  // Group g0 + j uses LDS stage (j + count) % 2, so that after an optional
  // lone first group (odd count) the loop runs in (stage 0, stage 1) pairs.
  const int count = g1 - g0;
  const int st0 = count & 1;
#pragma unroll
  for (int i = 0; i < 8; ++i) issue_x_one(g0, st0, i);
  load_w(g0, wn, sn);
  // the low-rank branch's loads go out behind the first group's, so that
  // their latencies overlap (32760 x 5120 x 5120, r = 32: 1558 -> 1504 us for
  // the fused call); it still adds into acc before the K loop
  if (lowrank && args.t != nullptr) {
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
    const int gn = min(g + 1, g1 - 1);
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
  int g = g0;
  if (st0 == 1) group(g++, I1{});
  for (; g < g1; g += 2) {
    group(g, I0{});
    group(g + 1, I1{});
  }
}

// Epilogue of tile (tm, tn): each 32 x 32 block leaves through a 5 KB
// scratch per wave in LDS as 16-byte pieces of rows.  Every wave must be done
// with LDS before it is called (a barrier after large_accumulate).
__device__ __forceinline__ void large_store(const GemmArgs& args, int tm, int tn,
                                            const f32x16 (&acc)[kBM / 32], uint8_t* lds) {
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  float* scratch = reinterpret_cast<float*>(lds + wave * kEpiScratch);
  const bool vec = epi_vec_ok(args.y, args.n, args.out_bf16 != 0);
  const int m0 = tm * kBM, nw0 = tn * kBN;
#pragma unroll
  for (int rb = 0; rb < kBM / 32; ++rb) {
    if (args.out_bf16)
      store_block32<true>(acc[rb], scratch, args.y, args.m, args.n, m0 + rb * 32, nw0 + wave * 32, vec);
    else
      store_block32<false>(acc[rb], scratch, args.y, args.m, args.n, m0 + rb * 32, nw0 + wave * 32, vec);
  }
}

__device__ __forceinline__ void zero_acc(f32x16 (&acc)[kBM / 32]) {
#pragma unroll
  for (int rb = 0; rb < kBM / 32; ++rb)
#pragma unroll
    for (int i = 0; i < 16; ++i) acc[rb][i] = 0.f;
}

// One whole 256 x 256 output tile (tile index `tile`).  Kernels:
// gemm_large_kernel (one product) and gemm_grouped_large_kernel (several
// products in one launch).
template <int B>
__device__ __forceinline__ void large_tile(const GemmArgs& args, int tile, uint8_t* lds) {
  int tm, tn;
  tile_coords(tile, args.tiles_m, args.tiles_n, tm, tn);
  f32x16 acc[kBM / 32];
  zero_acc(acc);
  large_accumulate<B>(args, tm, tn, 0, args.k / kGroup, true, acc, lds);
  __syncthreads();
  large_store(args, tm, tn, acc, lds);
}

template <int B>
__global__ __launch_bounds__(512, 1) void gemm_large_kernel(GemmArgs args) {
  __shared__ __attribute__((aligned(1024))) uint8_t lds[2 * kLdsStage];
  large_tile<B>(args, blockIdx.x, lds);
}

// ---------------------------------------------------------------------------
// K2n: large-M GEMM with 256 x 192 tiles, for outputs that 256 x 256 tiles
// cover with compute units left idle (4096 x 3072: 192 tiles of 256 x 256 for
// 256 units, 256 tiles of 256 x 192).  Workgroup = 4 waves, one per SIMD;
// wave w owns columns [48w, 48w + 48) for all 256 rows as three column blocks
// of 16, so every packed weight is still dequantized once per workgroup and
// each A fragment feeds three MFMAs.  MFMA v_mfma_f32_16x16x32_bf16: A = X
// rows (LDS), B = dequantized weights (registers), 192 accumulators per lane.
// K index inside a group: k-step j (0..3), lane quarter q = lane / 16,
// element e uses input 32q + 8j + e, for both operands.  X goes HBM -> LDS
// as in K2 (64 KB stages, double-buffered; row r holds 16 chunks of 16 bytes,
// logical chunk c in slot c ^ (r & 15)); the A fragment of lane (row r,
// quarter q) at k-step j is chunk 4q + j.  Lane (column lr = lane % 16,
// quarter q) of column block c streams the chunk of codes 32q .. 32q + 31 of
// column 48w + 16c + lr, one group ahead, and dequantizes it in the plus-one
// form (as dequant8_p1).
// ---------------------------------------------------------------------------
constexpr int kBN192 = 192;
constexpr int kEpi48Stride = 52;     // floats per scratch row (48 + 4: conflict-free writes)

template <int B>
__device__ __forceinline__ void n192_tile(const GemmArgs& args, int tm, int tn, uint8_t* lds) {
  constexpr int RB = kBM / 16;          // 16 row blocks of 16
  constexpr int CB = 3;                 // column blocks of 16 per wave
  constexpr int KS = 4;                 // k-steps of 32 per group
  constexpr int STEPS = KS * RB;        // 64 steps of three MFMAs
  constexpr int LA = 3;                 // A-operand look-ahead, in steps
  constexpr int RING = 4;
  constexpr int HAND = STEPS - LA;      // step of the group hand-over (barrier)
  constexpr int JOBS = CB * 4;          // dequantization jobs (bf16 pairs) per k-step
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int lane = threadIdx.x & 63;
  const int lr = lane & 15, lq = lane >> 4;
  const int m0 = tm * kBM;
  const int nw0 = tn * kBN192;
  const int K = args.k;
  const int G = K / kGroup;
  const uint32_t row_bytes = (uint32_t)K * B / 8;
  const uint32_t xrow_bytes = (uint32_t)K * 2;
  const int m_valid = min(kBM, args.m - m0);
  const int n_valid = min(kBN192, args.n - nw0);
  // Rows past M / columns past N read as zeros (their results are not stored).
  const rsrc_t rx = make_rsrc(args.x + (int64_t)m0 * K, (uint32_t)m_valid * xrow_bytes);
  const rsrc_t rw = make_rsrc(args.packed + (int64_t)nw0 * row_bytes, (uint32_t)n_valid * row_bytes);
  const rsrc_t rs = make_rsrc(args.scales + (int64_t)nw0 * G, (uint32_t)n_valid * G * 4);

  // X -> LDS.  DMA instruction i (0..15) of wave w fills 1 KB block 16w + i:
  // rows 64w + 4i + lane/16, slot lane%16, holding logical chunk slot ^ (row & 15).
  uint32_t xoff[4];
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const int r = wave * 64 + 4 * j + (lane >> 4);
    const int c = (lane & 15) ^ (r & 15);
    xoff[j] = (uint32_t)r * xrow_bytes + (uint32_t)c * 16;
  }
  auto issue_x_one = [&](int g, int stage, int i) {
    uint8_t* base = lds + stage * kLdsStage + wave * 16 * 1024;
    __builtin_amdgcn_raw_ptr_buffer_load_lds(rx, (lds_ptr_t)(base + i * 1024), 16,
                                             xoff[i & 3] + (uint32_t)(i >> 2) * 16 * xrow_bytes,
                                             (uint32_t)g * kGroup * 2, 0, 0);
  };

  // Packed chunks and scales of the lane's three columns.
  const uint32_t ncol = (uint32_t)(wave * 48 + lr);
  const uint32_t woff = ncol * row_bytes + (uint32_t)lq * 4 * B;
  const uint32_t soffs = ncol * (uint32_t)G * 4;
  auto load_w = [&](int g, uint32_t (&w)[CB][B], float (&s)[CB]) {
#pragma unroll
    for (int c = 0; c < CB; ++c) {
      load_chunk_buf<B>(rw, woff + (uint32_t)c * 16 * row_bytes, (uint32_t)g * 16 * B, w[c]);
      s[c] = __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(
                                           rs, soffs + (uint32_t)c * 16 * G * 4, (uint32_t)g * 4, 0));
    }
  };

  // A operand of step u (k-step u/16, row block u%16) from an LDS stage.
  uint32_t aoff[KS];
#pragma unroll
  for (int j = 0; j < KS; ++j) aoff[j] = (uint32_t)(lr * 256 + (((4 * lq + j) ^ lr) * 16));
  auto read_a = [&](int stage, int u) -> bf16x8 {
    return *reinterpret_cast<const bf16x8*>(lds + stage * kLdsStage + (u & 15) * 4096 + aoff[u >> 4]);
  };

  f32x4 acc[RB][CB];
#pragma unroll
  for (int rb = 0; rb < RB; ++rb)
#pragma unroll
    for (int c = 0; c < CB; ++c) acc[rb][c] = f32x4{0.f, 0.f, 0.f, 0.f};

  uint32_t wc[CB][B], wn[CB][B], be1[CB][B];
  float sc[CB], sn[CB], nsh[CB];
  uint32_t ev[CB], od[CB];              // 4-bit: the chunk dword's codes plus one, as bytes
  bf16x8 ring[RING];
  u32x4 bc[CB], bnx[CB];

  auto take_next_weights = [&]() {
#pragma unroll
    for (int c = 0; c < CB; ++c) {
#pragma unroll
      for (int j = 0; j < B; ++j) wc[c][j] = wn[c][j];
      sc[c] = sn[c];
      if constexpr (B != 4) plus_one_words<B>(wc[c], be1[c]);
      nsh[c] = -(float)(1 << (B - 1)) * sc[c];
    }
  };
  // dequantization job (chunk c, bf16 pair p) of k-step ks: codes 8ks + 2p, 8ks + 2p + 1
  auto dq_job = [&](int c, int p, int ks) {
    float a, b;
    if constexpr (B == 4) {
      if (p == 0) {
        const uint32_t x1 = wc[c][ks] + 0x11111111u;
        ev[c] = (x1 >> 4) & 0x0F0F0F0Fu;
        od[c] = x1 & 0x0F0F0F0Fu;
        // keep the masked words (two bytes per conversion below)
        asm("" : "+v"(ev[c]), "+v"(od[c]));
      }
      const f32x2 fa = (p >> 1) ? small_bytes_f32<1>(ev[c]) : small_bytes_f32<0>(ev[c]);
      const f32x2 fb = (p >> 1) ? small_bytes_f32<1>(od[c]) : small_bytes_f32<0>(od[c]);
      a = (p & 1) ? fa.y : fa.x;
      b = (p & 1) ? fb.y : fb.x;
    } else {
      a = (float)chunk_code_p1<B>(be1[c], 8 * ks + 2 * p);
      b = (float)chunk_code_p1<B>(be1[c], 8 * ks + 2 * p + 1);
    }
    bnx[c][p] = pack_bf16x2(__builtin_fmaf(a, sc[c], nsh[c]), __builtin_fmaf(b, sc[c], nsh[c]));
  };

#pragma unroll
  for (int i = 0; i < 16; ++i) issue_x_one(0, 0, i);
  load_w(0, wn, sn);
  // the low-rank branch behind the first group's loads, as in K2
  // (4096 x 3072 x 3072, r = 32: 87.6 -> 84.3 us for the fused call)
  if (args.t != nullptr) {
    // acc = T * lora_up^T over the rank dimension, 32 at a time (zero-padded).
    const int R = args.r;
    const bf16x8 zero = __builtin_bit_cast(bf16x8, u32x4{0u, 0u, 0u, 0u});
    for (int j0 = 0; j0 < R; j0 += 32) {
      const int kk = j0 + 8 * lq;
      const bool kok = kk < R;
      const int kc = min(kk, R - 8);
      bf16x8 bl[CB];
#pragma unroll
      for (int c = 0; c < CB; ++c) {
        const int n = min(nw0 + (int)ncol + 16 * c, args.n - 1);
        const bf16x8 v = *reinterpret_cast<const bf16x8*>(args.lora_up + (int64_t)n * R + kc);
        bl[c] = kok ? v : zero;
      }
#pragma unroll
      for (int rb = 0; rb < RB; ++rb) {
        const int m = min(m0 + rb * 16 + lr, args.m - 1);
        const bf16x8 tv = *reinterpret_cast<const bf16x8*>(args.t + (int64_t)m * R + kc);
        const bf16x8 a = kok ? tv : zero;
#pragma unroll
        for (int c = 0; c < CB; ++c) acc[rb][c] = mfma16x16x32(a, bl[c], acc[rb][c]);
      }
    }
  }
  __builtin_amdgcn_s_waitcnt(0);
  __syncthreads();
  take_next_weights();
#pragma unroll
  for (int u = 0; u < LA; ++u) ring[u % RING] = read_a(0, u);
#pragma unroll
  for (int j = 0; j < JOBS; ++j) dq_job(j >> 2, j & 3, 0);
#pragma unroll
  for (int c = 0; c < CB; ++c) bc[c] = bnx[c];

  // One 128-group: 64 steps (4 k-steps x 16 row blocks), three MFMAs each.
  // Every step index is a compile-time constant, so the operand ring and the
  // dequantization schedule are static:
  //   steps 0..15   one X DMA instruction each (next group -> idle stage)
  //   step 16       packed chunks + scales of the next group
  //   every step    one LDS read LA steps ahead; on row blocks 0..11 one
  //                 dequantization job for the next k-step; 3 MFMAs
  //   end of ks = 2 switch to the next group's weights (their loads landed)
  //   step HAND     barrier: the next group's X is in LDS, this stage is free
  // The last group's "next group" is itself (clamped), fetched into the idle
  // stage and never used.
  auto group = [&](int g, auto stage_tag) {
    constexpr int ST = decltype(stage_tag)::value;
    const int gn = min(g + 1, G - 1);
    auto step = [&]<int T>(std::integral_constant<int, T>) {
      constexpr int ks = T >> 4, rb = T & 15;
      if constexpr (T < 16) issue_x_one(gn, ST ^ 1, T);
      if constexpr (T == 16) load_w(gn, wn, sn);
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
      if constexpr (rb < JOBS) dq_job(rb >> 2, rb & 3, (ks + 1) & 3);
#pragma unroll
      for (int c = 0; c < CB; ++c)
        acc[rb][c] = mfma16x16x32(ring[T % RING], __builtin_bit_cast(bf16x8, bc[c]), acc[rb][c]);
      if constexpr (rb == RB - 1) {
#pragma unroll
        for (int c = 0; c < CB; ++c) bc[c] = bnx[c];
        if constexpr (ks == KS - 2) take_next_weights();
      }
      // the VALU work rides in the shadow of the three MFMAs (two VALU
      // instructions after each: 1-2% faster than three, in interleaved timings)
      __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
      __builtin_amdgcn_sched_group_barrier(0x002, 2, 0);
      __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
      __builtin_amdgcn_sched_group_barrier(0x002, 2, 0);
      __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
      __builtin_amdgcn_sched_group_barrier(0x002, 2, 0);
      __builtin_amdgcn_sched_barrier(0);
    };
    [&]<int... T>(std::integer_sequence<int, T...>) {
      (step(std::integral_constant<int, T>{}), ...);
    }(std::make_integer_sequence<int, STEPS>{});
  };

  using I0 = std::integral_constant<int, 0>;
  using I1 = std::integral_constant<int, 1>;
  int g = 0;
  for (; g + 1 < G; g += 2) {
    group(g, I0{});
    group(g + 1, I1{});
  }
  if (g < G) group(g, I0{});
  __syncthreads();

  // Epilogue: two row blocks (32 x 48) at a time through a per-wave scratch
  // in LDS, leaving as 16-byte pieces of rows.
  float* scratch = reinterpret_cast<float*>(lds + wave * 32 * kEpi48Stride * 4);
  const bool bf = args.out_bf16 != 0;
  const bool vec = epi_vec_ok(args.y, args.n, bf);
  const int col0 = nw0 + wave * 48;
#pragma unroll
  for (int rp = 0; rp < RB / 2; ++rp) {
#pragma unroll
    for (int h = 0; h < 2; ++h)
#pragma unroll
      for (int c = 0; c < CB; ++c)
#pragma unroll
        for (int i = 0; i < 4; ++i)
          scratch[(16 * h + 4 * lq + i) * kEpi48Stride + 16 * c + lr] = acc[2 * rp + h][c][i];
    __builtin_amdgcn_s_waitcnt(0xC07F);                    // lgkmcnt(0)
    __builtin_amdgcn_wave_barrier();
    const int W = bf ? 8 : 4;                              // values per 16-byte piece
    const int per_row = 48 / W;
    const int pieces = 32 * per_row;
    // A 32 x 48 block wholly inside Y, with 16-byte-aligned rows, needs no
    // per-lane checks: one branch on a uniform condition instead of a
    // divergent one per piece (4096 x 3072 x 3072: 70.5 -> 67.1 us)
    if (vec && m0 + 32 * rp + 32 <= args.m && col0 + 48 <= args.n) {
      if (bf) {
#pragma unroll
        for (int i = 0; i < 3; ++i) {
          const int q = lane + 64 * i, row = q / 6, cc = (q - row * 6) * 8;
          const float* src = scratch + row * kEpi48Stride + cc;
          const f32x4 lo = *reinterpret_cast<const f32x4*>(src);
          const f32x4 hi = *reinterpret_cast<const f32x4*>(src + 4);
          __bf16 v[8] = {(__bf16)lo[0], (__bf16)lo[1], (__bf16)lo[2], (__bf16)lo[3],
                         (__bf16)hi[0], (__bf16)hi[1], (__bf16)hi[2], (__bf16)hi[3]};
          store_out16(static_cast<__bf16*>(args.y) + (int64_t)(m0 + 32 * rp + row) * args.n + col0 + cc,
                      __builtin_bit_cast(u32x4, v));
        }
      } else {
#pragma unroll
        for (int i = 0; i < 6; ++i) {
          const int q = lane + 64 * i, row = q / 12, cc = (q - row * 12) * 4;
          const f32x4 t = *reinterpret_cast<const f32x4*>(scratch + row * kEpi48Stride + cc);
          store_out16(static_cast<float*>(args.y) + (int64_t)(m0 + 32 * rp + row) * args.n + col0 + cc,
                      __builtin_bit_cast(u32x4, t));
        }
      }
      __builtin_amdgcn_wave_barrier();
      continue;
    }
    for (int q = lane; q < pieces; q += 64) {
      const int row = q / per_row, cc = (q - row * per_row) * W;
      const int gr = m0 + 32 * rp + row, gc = col0 + cc;
      if (gr >= args.m || gc >= args.n) continue;
      const float* src = scratch + row * kEpi48Stride + cc;
      const int64_t base = (int64_t)gr * args.n + gc;
      if (bf) {
        const f32x4 lo = *reinterpret_cast<const f32x4*>(src);
        const f32x4 hi = *reinterpret_cast<const f32x4*>(src + 4);
        __bf16 v[8] = {(__bf16)lo[0], (__bf16)lo[1], (__bf16)lo[2], (__bf16)lo[3],
                       (__bf16)hi[0], (__bf16)hi[1], (__bf16)hi[2], (__bf16)hi[3]};
        __bf16* dst = static_cast<__bf16*>(args.y) + base;
        if (vec && gc + 8 <= args.n) {
          store_out16(dst, __builtin_bit_cast(u32x4, v));
        } else {
          for (int e = 0; e < 8 && gc + e < args.n; ++e) dst[e] = v[e];
        }
      } else {
        const f32x4 t = *reinterpret_cast<const f32x4*>(src);
        float* dst = static_cast<float*>(args.y) + base;
        if (vec && gc + 4 <= args.n) {
          store_out16(dst, __builtin_bit_cast(u32x4, t));
        } else {
          for (int e = 0; e < 4 && gc + e < args.n; ++e) dst[e] = t[e];
        }
      }
    }
    __builtin_amdgcn_wave_barrier();
  }
}

template <int B>
__global__ __launch_bounds__(256, 1) void gemm_n192_kernel(GemmArgs args) {
  __shared__ __attribute__((aligned(1024))) uint8_t lds[2 * kLdsStage];
  int tm, tn;
  // 2 tile rows per column strip: at 4096 x 3072 each XCD then takes 2 tile
  // rows x all 16 tile columns and reads its X row strips once (4 rows x 8
  // columns read every strip on 2 XCDs: 96 MB of HBM traffic per launch
  // against 90 MB)
  tile_coords<2>(blockIdx.x, args.tiles_m, args.tiles_n, tm, tn);
  n192_tile<B>(args, tm, tn, lds);
}

// ---------------------------------------------------------------------------
// K2sk: the large-M product with K split across workgroups, for outputs whose
// 256 x 256 tiles would fill the compute units unevenly.  At most one
// workgroup per compute unit, all resident at once.  Two assignments:
//   * split-K (split > 1, few tiles): workgroup u takes K chunk u / tiles
//     (of `split` equal chunks) of tile u % tiles, so the workgroups of one
//     moment read the same K range of the operands (they share L2 the way
//     whole tiles do);
//   * stream-K (split == 0): workgroup w runs on XCD w % 8 (the dispatcher's
//     round robin); the tiles are split into 8 contiguous sets, one per XCD,
//     and each XCD's (tile, 128-group) iterations into equal contiguous
//     ranges, one per workgroup of that XCD in order of w / 8.  A range holds
//     at most one tile's tail (it starts inside a tile), whole tiles, and at
//     most one tile's head (it ends inside a tile).
// Split-K: every chunk writes its partial tile to its workgroup's slot of the
// workspace and sets its flag to this launch's epoch; then the chunks of a
// tile wait for one another's flags and each adds up, in chunk order, and
// stores a share of the tile's 32 x 32 blocks (the reduction is spread over
// the tile's workgroups).  The grid is at most one workgroup per compute unit
// (128 KB of LDS each), so all of them are resident once dispatched, and each
// publishes before it waits.
// Stream-K: a piece that ends before the tile's last group publishes its
// partial sums the same way; the piece holding the tile's last group waits
// for the flags of the workgroups holding the tile's other groups, adds their
// partial sums in workgroup order and stores the tile.  Those workgroups have
// smaller ids (the dispatcher starts them first) and publish before they wait
// for anything.
// Either way the sums are added in a fixed order, so results do not depend on
// timing.  Each wait is also bounded (a flag that never comes, which a correct
// caller never causes, ends it after about a second with a wrong tile instead
// of a hang).  Flags hold a per-launch epoch (never zero, drawn by the host
// from a random start), so the workspace needs no clearing.
// ---------------------------------------------------------------------------
struct StreamK {
  float* partials;                 // grid x 65536 floats, accumulator layout
  unsigned long long* flags;       // grid flags
  unsigned long long epoch;
  int wpx;                         // stream-K: workgroups per XCD (grid = 8 wpx)
  int split;                       // split-K: K chunks per tile (grid = split x tiles); 0: stream-K
};
constexpr int kSkXcds = 8;
constexpr int kSkSlotFloats = kBM * kBN;
constexpr unsigned kSkSpinLimit = 1u << 20;
// The exchange bypasses the cache maintenance of fences (an agent-scope
// acquire invalidates the whole XCD L2, which the other workgroups of that XCD
// are streaming X and weights through): the partial sums are written and read
// with device-scope coherent buffer accesses (cache policy SC1) and the flags
// are relaxed agent-scope atomics.  A writer's partial stores have completed
// (s_waitcnt, then the workgroup barrier) before its flag is stored; a reader
// issues its partial loads only after it has seen the flag.
constexpr int kSkCoherent = 16;   // SC1
constexpr int kSkMaxSplit = 8;    // K chunks per tile in split-K

template <int B>
__global__ __launch_bounds__(512, 1) void gemm_streamk_kernel(GemmArgs args, StreamK sk) {
  __shared__ __attribute__((aligned(1024))) uint8_t lds[2 * kLdsStage];
  const int w = blockIdx.x;
  const int G = args.k / kGroup;
  const int tiles = args.tiles_m * args.tiles_n;
  const bool split_k = sk.split > 0;
  // stream-K: this XCD's tiles and this workgroup's iteration range
  const int xcd = w % kSkXcds, l = w / kSkXcds;
  const int t_lo = split_k ? 0 : (int)((int64_t)xcd * tiles / kSkXcds);
  const int t_hi = split_k ? 0 : (int)((int64_t)(xcd + 1) * tiles / kSkXcds);
  const int64_t I = (int64_t)(t_hi - t_lo) * G;
  auto start = [&](int ll) { return (int64_t)(I * ll / sk.wpx); };
  int nseg, tf = 0, tl = 0, a_f = 0, b_l = G;
  bool head_last = false;
  if (split_k) {
    nseg = 1;
  } else {
    const int64_t i0 = start(l), i1 = start(l + 1);
    if (i0 >= i1) return;
    tf = (int)(i0 / G); tl = (int)((i1 - 1) / G);                  // first, last tile (XCD-relative)
    a_f = (int)(i0 % G); b_l = (int)((i1 - 1) % G) + 1;
    head_last = b_l < G && tl != tf;                                // ends inside another tile
    nseg = tl - tf + 1;
  }
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int lane = threadIdx.x & 63;
  // a slot holds the 256 x 256 partial tile in the accumulator layout: wave
  // w's 32 KB, then (row block, quarter) pieces of 1 KB, 16 bytes per lane
  const uint32_t slot_voff = (uint32_t)wave * 32768u + (uint32_t)lane * 16u;
  auto slot_rsrc = [&](int wi) {
    return make_rsrc(sk.partials + (int64_t)wi * kSkSlotFloats, (uint32_t)(kSkSlotFloats * 4));
  };

  for (int s = 0; s < nseg; ++s) {
    int tm, tn, a, b, n_contrib, c_first;
    if (split_k) {
      const int c = w / tiles, t = w % tiles;
      tile_coords(t, args.tiles_m, args.tiles_n, tm, tn);
      a = (int)((int64_t)c * G / sk.split);
      b = (int)((int64_t)(c + 1) * G / sk.split);
      n_contrib = c;                    // chunks 0 .. c-1 of this tile: workgroups c' tiles + t
      c_first = t;
    } else {
      // order: the head of the last tile, the whole tiles, the first tile
      int t;
      if (head_last) t = s == 0 ? tl : (s == nseg - 1 ? tf : tf + s);
      else t = s == nseg - 1 ? tf : tf + 1 + s;
      t = __builtin_amdgcn_readfirstlane(t);
      a = t == tf ? a_f : 0;
      b = t == tl ? b_l : G;
      tile_coords_range(t_lo + t, args.tiles_m, args.tiles_n, tm, tn);
      // earlier workgroups of this XCD holding groups of this tile: c_first .. l-1
      const int64_t it0 = (int64_t)t * G;
      int c0 = l - 1;
      while (c0 > 0 && start(c0) > it0) --c0;
      c_first = c0;
      n_contrib = l - c0;
    }
    f32x16 acc[kBM / 32];
    zero_acc(acc);
    large_accumulate<B>(args, tm, tn, a, b, a == 0, acc, lds);
    __syncthreads();
    if (split_k) {
      // every chunk publishes its partial tile, then reduces and stores the
      // 32 x 32 blocks (wave, row block) numbered chunk, chunk + split, ...
      // of the tile from all `split` slots in chunk order
      const rsrc_t ro = slot_rsrc(w);
#pragma unroll
      for (int rb = 0; rb < kBM / 32; ++rb)
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          typedef float f4 __attribute__((ext_vector_type(4)));
          typedef uint32_t u4 __attribute__((ext_vector_type(4)));
          const f4 v = {acc[rb][4 * q], acc[rb][4 * q + 1], acc[rb][4 * q + 2], acc[rb][4 * q + 3]};
          __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(u4, v), ro, slot_voff,
                                                 (uint32_t)((rb * 4 + q) * 1024), kSkCoherent);
        }
      __builtin_amdgcn_s_waitcnt(0);
      __syncthreads();
      if (threadIdx.x == 0)
        __hip_atomic_store(&sk.flags[w], sk.epoch, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      const int chunk = w / tiles;
      for (int c = 0; c < sk.split; ++c) {
        if (c == chunk) continue;
        unsigned spins = 0;
        while (__hip_atomic_load(&sk.flags[c * tiles + c_first], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) !=
                   sk.epoch && ++spins < kSkSpinLimit)
          __builtin_amdgcn_s_sleep(1);
      }
      __builtin_amdgcn_s_waitcnt(0);
      float* scratch = reinterpret_cast<float*>(lds + wave * kEpiScratch);
      const bool vec = epi_vec_ok(args.y, args.n, args.out_bf16 != 0);
      const uint32_t lane_off = (uint32_t)lane * 16u;
      for (int piece = chunk + sk.split * wave; piece < 8 * (kBM / 32); piece += sk.split * 8) {
        const int pw = piece / (kBM / 32), prb = piece % (kBM / 32);   // block of wave pw, row block prb
        // every chunk's block in flight at once (chunks past `split` read
        // nothing: their offset lies past the resource and returns zeros),
        // then added in chunk order
        typedef uint32_t u4 __attribute__((ext_vector_type(4)));
        u4 r[kSkMaxSplit][4];
#pragma unroll
        for (int c = 0; c < kSkMaxSplit; ++c) {
          const bool live = c < sk.split;
          const rsrc_t ri = slot_rsrc((live ? c : 0) * tiles + c_first);
#pragma unroll
          for (int q = 0; q < 4; ++q)
            r[c][q] = __builtin_amdgcn_raw_buffer_load_b128(ri, live ? lane_off : 0x80000000u,
                                                             (uint32_t)(pw * 32768 + (prb * 4 + q) * 1024),
                                                             kSkCoherent);
        }
        f32x16 v16;
#pragma unroll
        for (int i = 0; i < 16; ++i) v16[i] = 0.f;
#pragma unroll
        for (int c = 0; c < kSkMaxSplit; ++c)
#pragma unroll
          for (int q = 0; q < 4; ++q) {
            const f32x4 f = __builtin_bit_cast(f32x4, r[c][q]);
            v16[4 * q] += f[0]; v16[4 * q + 1] += f[1]; v16[4 * q + 2] += f[2]; v16[4 * q + 3] += f[3];
          }
        if (args.out_bf16)
          store_block32<true>(v16, scratch, args.y, args.m, args.n, tm * kBM + prb * 32, tn * kBN + pw * 32, vec);
        else
          store_block32<false>(v16, scratch, args.y, args.m, args.n, tm * kBM + prb * 32, tn * kBN + pw * 32, vec);
      }
      continue;
    }
    if (b < G) {
      // partial: publish this workgroup's sums of the tile
      const rsrc_t ro = slot_rsrc(w);
#pragma unroll
      for (int rb = 0; rb < kBM / 32; ++rb)
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          typedef float f4 __attribute__((ext_vector_type(4)));
          typedef uint32_t u4 __attribute__((ext_vector_type(4)));
          const f4 v = {acc[rb][4 * q], acc[rb][4 * q + 1], acc[rb][4 * q + 2], acc[rb][4 * q + 3]};
          __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(u4, v), ro, slot_voff,
                                                 (uint32_t)((rb * 4 + q) * 1024), kSkCoherent);
        }
      __builtin_amdgcn_s_waitcnt(0);
      __syncthreads();
      if (threadIdx.x == 0)
        __hip_atomic_store(&sk.flags[w], sk.epoch, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      continue;
    }
    if (a > 0) {
      // the tile's last piece: add the partial sums of its other pieces
      for (int j = 0; j < n_contrib; ++j) {
        int wc;
        if (split_k) {
          wc = j * tiles + c_first;
        } else {
          const int c = c_first + j;
          if (start(c) >= start(c + 1)) continue;                  // an empty range publishes nothing
          wc = c * kSkXcds + xcd;
        }
        unsigned spins = 0;
        while (__hip_atomic_load(&sk.flags[wc], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) != sk.epoch &&
               ++spins < kSkSpinLimit)
          __builtin_amdgcn_s_sleep(1);
        __builtin_amdgcn_s_waitcnt(0);
        const rsrc_t ri = slot_rsrc(wc);
#pragma unroll
        for (int rb = 0; rb < kBM / 32; ++rb)
#pragma unroll
          for (int q = 0; q < 4; ++q) {
            typedef uint32_t u4 __attribute__((ext_vector_type(4)));
            const u4 r = __builtin_amdgcn_raw_buffer_load_b128(ri, slot_voff, (uint32_t)((rb * 4 + q) * 1024),
                                                                kSkCoherent);
            const f32x4 v = __builtin_bit_cast(f32x4, r);
            acc[rb][4 * q] += v[0]; acc[rb][4 * q + 1] += v[1];
            acc[rb][4 * q + 2] += v[2]; acc[rb][4 * q + 3] += v[3];
          }
      }
    }
    large_store(args, tm, tn, acc, lds);
    __syncthreads();
  }
}

// ---------------------------------------------------------------------------
// K3: small-M GEMM (16 < M <= 64; M <= 16 when the skinny kernel below
// does not apply): a bandwidth kernel.
// Workgroup = NC x NK waves.  Wave (c, h) owns column block c (16 columns of
// the workgroup's 16*NC) and K split h (a contiguous range of 128-groups).
//   * X: for each group, the 16*RB x 128 bf16 slice of a K split is loaded
//     into registers (16 bytes per lane per 1 KB piece, the pieces shared out
//     among the NC waves of that split), written to an LDS ring and read back
//     as MFMA A operands by all NC waves.  Rows past M read as zeros.
//   * packed weights: each lane's chunk (B dwords) and scale in a register
//     ring; the X slice and the weights of step j + D are loaded together at
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
// K split across workgroups for M <= 16 (one row block): workgroup (wg,
// part) runs groups [part G / parts, (part + 1) G / parts) of its column
// blocks.  Every part but the last publishes each column block's 16 x 16
// partial sum (1 KB, the accumulator layout) to its slot and sets its flag;
// the last part waits for the flags of the earlier parts (smaller workgroup
// ids, dispatched before it), adds the partial sums in part order and its
// own last (the same order on every call), and stores the result.  The
// exchange uses the device-coherent accesses and epoch flags of StreamK.
struct SmallSplit {
  float* partials;                 // column blocks x parts x 256 floats
  unsigned long long* flags;       // column blocks x parts
  unsigned long long epoch;
  int parts;                       // 1: K is not split
};
constexpr int kSmallMaxParts = 8;

template <int B, int RB, int NC, int NK>
__device__ __forceinline__ void small_body(const GemmArgs& args, int wg, SmallLds<RB, NC, NK>& L,
                                           const SmallSplit& sp = SmallSplit{nullptr, nullptr, 0, 1},
                                           int part = 0) {
  // X slices and packed weights of step j + D are loaded into registers at
  // step j (rings of S = D + 1 slots); at step j each wave writes its share of
  // X(j) to the LDS slot, and one LDS barrier hands the slot to the other
  // column waves.  Every wait is the compiler's own (register dependences), so
  // no wait depends on the order in which the loads were issued.
  constexpr int XSLOT = SmallLds<RB, NC, NK>::XSLOT;
  constexpr int S = SmallLds<RB, NC, NK>::S;
  constexpr int D = S - 1;                    // steps in flight
  constexpr int PIECES = XSLOT / 1024;        // 1 KB pieces per slice (64 lanes x 16 bytes)
  static_assert(PIECES % NC == 0, "the slice must split evenly over the column waves");
  constexpr int ND = PIECES / NC;             // pieces per wave per group

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
  // this workgroup's part of K, and this wave's share of it
  const int ga = (int)((int64_t)part * G / sp.parts), gb = (int)((int64_t)(part + 1) * G / sp.parts);
  const int gp = gb - ga;
  const int g_begin = ga + h * gp / NK, g_end = ga + (h + 1) * gp / NK;
  const int cnt = g_end - g_begin;
  const int steps = (gp + NK - 1) / NK;       // the same for every wave (barriers)
  const int g_last = cnt > 0 ? g_end - 1 : G - 1;
  const uint32_t row_bytes = (uint32_t)K * B / 8;

  // this wave's column (rows past N read as zeros through the resource bounds)
  const int n = min(n0 + c * 16 + lr, args.n - 1);
  const int n_valid = min(16 * NC, args.n - n0);
  const rsrc_t rw = make_rsrc(args.packed + (int64_t)n0 * row_bytes, (uint32_t)n_valid * row_bytes);
  const rsrc_t rs = make_rsrc(args.scales + (int64_t)n0 * G, (uint32_t)n_valid * G * 4);
  const uint32_t woff = (uint32_t)(c * 16 + lr) * row_bytes + (uint32_t)lq * 4 * B;
  const uint32_t soffs = (uint32_t)(c * 16 + lr) * (uint32_t)G * 4;

  // X piece d of this wave: 1 KB block c*ND + d of the slice, rows
  // 4*(c*ND+d) + lane/16; the lane's 16 bytes go to LDS position lane % 16 of
  // its row and hold logical chunk (lane % 16) ^ (row & 15) (conflict-free
  // operand reads).  Rows past M read zeros.
  const rsrc_t rx = make_rsrc(args.x, (uint32_t)args.m * (uint32_t)K * 2);
  typedef uint32_t u4 __attribute__((ext_vector_type(4)));
  u4 xr[S][ND];
  auto load_x = [&](int slot, int j) {
    const int g = min(g_begin + j, g_last);
#pragma unroll
    for (int d = 0; d < ND; ++d) {
      const int row = 4 * (c * ND + d) + (lane >> 4);
      const uint32_t voff = (uint32_t)row * (uint32_t)K * 2 + (uint32_t)(((lane & 15) ^ (row & 15)) * 16);
      xr[slot][d] = __builtin_amdgcn_raw_buffer_load_b128(rx, voff, (uint32_t)g * kGroup * 2, 0);
    }
  };
  auto write_x = [&](uint8_t* slot_base, int slot) {
    uint8_t* base = slot_base + (c * ND) * 1024 + lane * 16;
#pragma unroll
    for (int d = 0; d < ND; ++d) *reinterpret_cast<u4*>(base + d * 1024) = xr[slot][d];
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

  // Step j (ring slot j % S of the three rings): write this wave's share of
  // X(j) into LDS slot j % S, LDS barrier (every wave's share is there, and
  // every wave is done with step j - 1, so slot (j - 1) % S is free), load
  // X(j+D) and W(j+D) into register slot (j - 1) % S, compute step j.  Slot
  // j % S last held X(j - S), read at step j - S <= j - 2, which every wave
  // finished before the barrier of step j - 1.  The last steps (the tail)
  // load nothing: their loads would be for steps past the end.
  using std::integral_constant;
  auto step = [&]<int U, bool TAIL>(integral_constant<int, U>, std::bool_constant<TAIL>, int j) {
    write_x(xslot(integral_constant<int, U % S>{}), U % S);
    lds_barrier();
    if constexpr (!TAIL) {
      load_x((U + D) % S, j + D);
      load_w((U + D) % S, j + D);
    }
    if (j < cnt) compute(xslot(integral_constant<int, U % S>{}), U % S);
  };
  // prologue: steps 0..D-1
  [&]<int... J>(std::integer_sequence<int, J...>) {
    ((load_x(J, J), load_w(J, J)), ...);
  }(std::make_integer_sequence<int, D>{});
  // main loop: whole blocks of S steps (every ring index a constant)
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

  if constexpr (RB == 1) {
    if (sp.parts > 1) {
      typedef uint32_t u4 __attribute__((ext_vector_type(4)));
      const int cb = wg * NC + c;                           // column block of 16
      const rsrc_t rp = make_rsrc(sp.partials + (int64_t)cb * sp.parts * 256, (uint32_t)sp.parts * 1024u);
      if (part < sp.parts - 1) {
        __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(u4, acc[0]), rp, (uint32_t)lane * 16u,
                                               (uint32_t)part * 1024u, kSkCoherent);
        __builtin_amdgcn_s_waitcnt(0);
        if (lane == 0)
          __hip_atomic_store(&sp.flags[(int64_t)cb * sp.parts + part], sp.epoch, __ATOMIC_RELAXED,
                             __HIP_MEMORY_SCOPE_AGENT);
        return;
      }
      for (int q = 0; q < sp.parts - 1; ++q) {
        unsigned spins = 0;
        while (__hip_atomic_load(&sp.flags[(int64_t)cb * sp.parts + q], __ATOMIC_RELAXED,
                                 __HIP_MEMORY_SCOPE_AGENT) != sp.epoch &&
               ++spins < kSkSpinLimit)
          __builtin_amdgcn_s_sleep(1);
      }
      __builtin_amdgcn_s_waitcnt(0);
      // every earlier part's sums in flight at once (parts past the count read
      // nothing: their offset lies past the resource), then added in order
      u4 r[kSmallMaxParts - 1];
#pragma unroll
      for (int q = 0; q < kSmallMaxParts - 1; ++q)
        r[q] = __builtin_amdgcn_raw_buffer_load_b128(rp, q < sp.parts - 1 ? (uint32_t)lane * 16u : 0x80000000u,
                                                     (uint32_t)q * 1024u, kSkCoherent);
      f32x4 sum = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int q = 0; q < kSmallMaxParts - 1; ++q) {
        if (q < sp.parts - 1) {
          const f32x4 v = __builtin_bit_cast(f32x4, r[q]);
          sum[0] += v[0]; sum[1] += v[1]; sum[2] += v[2]; sum[3] += v[3];
        }
      }
      sum[0] += acc[0][0]; sum[1] += acc[0][1]; sum[2] += acc[0][2]; sum[3] += acc[0][3];
      acc[0] = sum;
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

// M <= 16 with K split across workgroups: workgroup id = wg * parts + part.
template <int B, int NC>
__global__ __launch_bounds__(64 * NC) void gemm_small_split_kernel(GemmArgs args, SmallSplit sp) {
  __shared__ SmallLds<1, NC, 1> L;
  const int wg = blockIdx.x / sp.parts, part = blockIdx.x - wg * sp.parts;
  small_body<B, 1, NC, 1>(args, wg, L, sp, part);
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

struct GroupArgs {
  GemmArgs g[kMaxGroup];
  int wg_start[kMaxGroup + 1];
  int bits[kMaxGroup];
  int kc[kMaxGroup];
  int count;
  int ncb;          // M <= 16 launch: column blocks of 16 per workgroup (1, 2 or 4)
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
// Workgroup = 4 waves over RR blocks of 16 token rows; waves split K in
// 32-wide steps; the 4 partials are summed through LDS in wave order, then
// rounded to bf16 once.
// ---------------------------------------------------------------------------
constexpr int kLowrankWaves = 4;

template <int RBLK, int RR>
__global__ __launch_bounds__(64 * kLowrankWaves) void lowrank_t_kernel(const __bf16* __restrict__ x,
                                                                       const __bf16* __restrict__ lora_down,
                                                                       __bf16* __restrict__ t, int m, int k,
                                                                       int r) {
  // RR blocks of 16 token rows per workgroup: every lora_down fragment a wave
  // loads feeds RR MFMAs, so lora_down (r x K, read whole by every workgroup)
  // costs 1/RR of its bytes per token row
  static_assert(RR * RBLK <= 8, "partial tiles in LDS: at most 32 KB");
  constexpr int NW = kLowrankWaves;
  __shared__ f32x4 red[NW][RR][RBLK][64];
  const int wave = threadIdx.x >> 6;
  const int lane = threadIdx.x & 63;
  const int lr = lane & 15, lq = lane >> 4;
  const int m0 = blockIdx.x * 16 * RR;
  const __bf16* xrow[RR];
#pragma unroll
  for (int i = 0; i < RR; ++i) xrow[i] = x + (int64_t)min(m0 + 16 * i + lr, m - 1) * k + 8 * lq;
  f32x4 acc[RR][RBLK];
#pragma unroll
  for (int i = 0; i < RR; ++i)
#pragma unroll
    for (int j = 0; j < RBLK; ++j) acc[i][j] = f32x4{0.f, 0.f, 0.f, 0.f};
  // U steps of this wave's K range per trip, their loads issued before the
  // first MFMA (the loop is bound by load latency otherwise); U by the loads
  // of one step
  constexpr int LPS = RR + RBLK;
  constexpr int U = LPS <= 3 ? 8 : (LPS <= 5 ? 4 : 2);
  const int steps = (k - wave * 32 + 32 * NW - 1) / (32 * NW);
  int st = 0;
  for (; st + U <= steps; st += U) {
    bf16x8 bv[U][RR], av[U][RBLK];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int k0 = wave * 32 + 32 * NW * (st + u);
#pragma unroll
      for (int i = 0; i < RR; ++i) bv[u][i] = *reinterpret_cast<const bf16x8*>(xrow[i] + k0);
#pragma unroll
      for (int j = 0; j < RBLK; ++j) {
        const int rr = j * 16 + lr;
        av[u][j] = load_bf16x8_or_zero(lora_down + (int64_t)min(rr, r - 1) * k + k0 + 8 * lq, rr < r);
      }
    }
#pragma unroll
    for (int u = 0; u < U; ++u)
#pragma unroll
      for (int i = 0; i < RR; ++i)
#pragma unroll
        for (int j = 0; j < RBLK; ++j) acc[i][j] = mfma16x16x32(av[u][j], bv[u][i], acc[i][j]);
  }
  for (; st < steps; ++st) {
    const int k0 = wave * 32 + 32 * NW * st;
    bf16x8 b[RR];
#pragma unroll
    for (int i = 0; i < RR; ++i) b[i] = *reinterpret_cast<const bf16x8*>(xrow[i] + k0);
#pragma unroll
    for (int j = 0; j < RBLK; ++j) {
      const int rr = j * 16 + lr;
      const bf16x8 a = load_bf16x8_or_zero(lora_down + (int64_t)min(rr, r - 1) * k + k0 + 8 * lq,
                                           rr < r);
#pragma unroll
      for (int i = 0; i < RR; ++i) acc[i][j] = mfma16x16x32(a, b[i], acc[i][j]);
    }
  }
#pragma unroll
  for (int i = 0; i < RR; ++i)
#pragma unroll
    for (int j = 0; j < RBLK; ++j) red[wave][i][j][lane] = acc[i][j];
  __syncthreads();
  // wave i (< RR) sums and stores row block i, the partials in wave order
  if (wave < RR) {
#pragma unroll
    for (int i = 0; i < RR; ++i) {
      if (i != wave) continue;
      const int mm = m0 + 16 * i + lr;
#pragma unroll
      for (int j = 0; j < RBLK; ++j) {
        f32x4 s = red[0][i][j][lane];
#pragma unroll
        for (int w = 1; w < NW; ++w) {
          const f32x4 v = red[w][i][j][lane];
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
}

// ---------------------------------------------------------------------------
// The pre-pass for few token rows, K split over workgroups.  With one
// workgroup per 16 rows, 16 tokens leave the whole pre-pass to one compute
// unit, which cannot keep enough misses in flight to read lora_down quickly.
// Workgroup (b, c) sums row block b over K chunk c (gpc whole groups) as the
// kernel above does and writes its float32 partial tile to part[c][row][j];
// lowrank_t_reduce_kernel then adds the chunks in chunk order and rounds to
// bf16 once, so the result repeats bit for bit.
// ---------------------------------------------------------------------------
template <int RBLK>
__global__ __launch_bounds__(64 * kLowrankWaves) void lowrank_t_part_kernel(const __bf16* __restrict__ x,
                                                                            const __bf16* __restrict__ lora_down,
                                                                            float* __restrict__ part, int m,
                                                                            int k, int r, int gpc) {
  constexpr int NW = kLowrankWaves;
  __shared__ f32x4 red[NW][RBLK][64];
  const int wave = threadIdx.x >> 6;
  const int lane = threadIdx.x & 63;
  const int lr = lane & 15, lq = lane >> 4;
  const int m0 = blockIdx.x * 16;
  const int c = blockIdx.y;
  const int kb = c * gpc * kGroup;                      // chunk start (< k)
  const int kl = min(gpc * kGroup, k - kb);             // chunk length, whole groups
  const __bf16* xrow = x + (int64_t)min(m0 + lr, m - 1) * k + kb + 8 * lq;
  const __bf16* lrow[RBLK];
#pragma unroll
  for (int j = 0; j < RBLK; ++j) lrow[j] = lora_down + (int64_t)min(j * 16 + lr, r - 1) * k + kb + 8 * lq;
  f32x4 acc[RBLK];
#pragma unroll
  for (int j = 0; j < RBLK; ++j) acc[j] = f32x4{0.f, 0.f, 0.f, 0.f};
  constexpr int U = 4;                                  // steps per batch of loads
  const int steps = (kl - wave * 32 + 32 * NW - 1) / (32 * NW);
  int st = 0;
  for (; st + U <= steps; st += U) {
    bf16x8 bv[U], av[U][RBLK];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int k0 = wave * 32 + 32 * NW * (st + u);
      bv[u] = *reinterpret_cast<const bf16x8*>(xrow + k0);
#pragma unroll
      for (int j = 0; j < RBLK; ++j) av[u][j] = load_bf16x8_or_zero(lrow[j] + k0, j * 16 + lr < r);
    }
#pragma unroll
    for (int u = 0; u < U; ++u)
#pragma unroll
      for (int j = 0; j < RBLK; ++j) acc[j] = mfma16x16x32(av[u][j], bv[u], acc[j]);
  }
  for (; st < steps; ++st) {
    const int k0 = wave * 32 + 32 * NW * st;
    const bf16x8 b = *reinterpret_cast<const bf16x8*>(xrow + k0);
#pragma unroll
    for (int j = 0; j < RBLK; ++j)
      acc[j] = mfma16x16x32(load_bf16x8_or_zero(lrow[j] + k0, j * 16 + lr < r), b, acc[j]);
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
      for (int w = 1; w < NW; ++w) {
        const f32x4 v = red[w][j][lane];
        s[0] += v[0]; s[1] += v[1]; s[2] += v[2]; s[3] += v[3];
      }
      const int rr = j * 16 + 4 * lq;
      if (mm < m && rr < r)
        *reinterpret_cast<f32x4*>(part + ((int64_t)c * m + mm) * r + rr) = s;
    }
  }
}

// T[i] = bf16(sum over chunks c in order of part[c][i]), four outputs a lane.
// (A template, as every kernel of this header, so that the units that
// include it share one definition.)
template <int V = 0>
__global__ __launch_bounds__(256) void lowrank_t_reduce_kernel(const float* __restrict__ part,
                                                               __bf16* __restrict__ t, int m, int r,
                                                               int chunks) {
  const int64_t q = (int64_t)blockIdx.x * 256 + threadIdx.x;
  const int64_t n4 = (int64_t)m * r / 4;
  if (q >= n4) return;
  f32x4 s = *reinterpret_cast<const f32x4*>(part + 4 * q);
  for (int c = 1; c < chunks; ++c) {
    const f32x4 v = *reinterpret_cast<const f32x4*>(part + (int64_t)c * m * r + 4 * q);
    s[0] += v[0]; s[1] += v[1]; s[2] += v[2]; s[3] += v[3];
  }
  u32x2 o = {pack_bf16x2(s[0], s[1]), pack_bf16x2(s[2], s[3])};
  *reinterpret_cast<u32x2*>(t + 4 * q) = o;
}

}  // namespace ddg
