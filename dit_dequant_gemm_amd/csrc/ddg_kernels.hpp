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
// IEEE float32 throughout: correctly rounded multiply and divide, round half
// to even, no fused operations (the file is compiled with -ffp-contract=off),
// subnormals kept.
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

  uint32_t out[B];
  uint64_t acc = 0;
  int nbits = 0, wo = 0;
#pragma unroll
  for (int i = 0; i < 32; ++i) {
    float q = __builtin_rintf(v[i] / step);
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
// K2: large-M GEMM.  Workgroup = 4 waves (256 threads), tile BM = 256 rows x
// BN = 4*WN columns; wave w owns columns [w*WN, (w+1)*WN) for all 256 rows,
// so every packed weight is dequantized exactly once per workgroup.
// K advances one 128-group per step:
//   * X[256 x 128] bf16 (64 KB) goes HBM -> LDS with global_load_lds_dwordx4,
//     double-buffered (2 x 64 KB).  LDS row r holds 16 chunks of 16 bytes;
//     logical chunk c sits in slot c ^ (r & 15) so that MFMA A-operand reads
//     are free of bank conflicts.
//   * each lane streams its packed chunk (B dwords) + scale for each of its
//     WN/16 columns straight to registers, one step ahead.
// MFMA v_mfma_f32_16x16x32_bf16.  The K index inside a group is permuted so
// that MFMA sub-step s, lane quarter lq, element e uses input
// 32*lq + 8*s + e: the A operand (X from LDS) and the B operand (dequantized
// codes) use the same permutation, so the dot products are unchanged.
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

template <int B, int CB>
__global__ __launch_bounds__(256, 1) void gemm_large_kernel(GemmArgs args) {
  constexpr int RB = kBM / 16;          // 16 row blocks of 16
  constexpr int LA = 6;                 // A-operand look-ahead, in MFMA steps
  constexpr int RING = 8;               // A-operand ring (64 steps per group = 8 laps)
  constexpr int WN = 16 * CB;
  constexpr int BN = 4 * WN;
  constexpr int HAND = 64 - LA;         // step of the group hand-over (barrier)
  __shared__ __attribute__((aligned(1024))) uint8_t lds[2 * kLdsStage];

  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int lane = threadIdx.x & 63;
  const int lr = lane & 15, lq = lane >> 4;
  int tm, tn;
  tile_coords(blockIdx.x, args.tiles_m, args.tiles_n, tm, tn);
  const int m0 = tm * kBM;
  const int nw0 = tn * BN;
  const int K = args.k;
  const int G = K / kGroup;
  const uint32_t row_bytes = (uint32_t)K * B / 8;
  const uint32_t xrow_bytes = (uint32_t)K * 2;
  const int m_valid = min(kBM, args.m - m0);
  const int n_valid = min(BN, args.n - nw0);
  // Rows past M / columns past N read as zeros (their results are not stored).
  const rsrc_t rx = make_rsrc(args.x + (int64_t)m0 * K, (uint32_t)m_valid * xrow_bytes);
  const rsrc_t rw = make_rsrc(args.packed + (int64_t)nw0 * row_bytes, (uint32_t)n_valid * row_bytes);
  const rsrc_t rs = make_rsrc(args.scales + (int64_t)nw0 * G, (uint32_t)n_valid * G * 4);

  // X -> LDS.  DMA instruction i of this wave fills 1 KB block wave*16+i: rows
  // 4*(wave*16+i) + lane/16, slot lane%16, holding logical chunk slot^(row&15).
  uint32_t xoff[4];
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const int r = wave * 64 + 4 * j + lq;
    const int c = (lane & 15) ^ (r & 15);
    xoff[j] = (uint32_t)r * xrow_bytes + (uint32_t)c * 16;
  }
  auto issue_x_one = [&](int g, int stage, int i) {
    uint8_t* base = lds + stage * kLdsStage + wave * 16 * 1024;
    __builtin_amdgcn_raw_ptr_buffer_load_lds(rx, (lds_ptr_t)(base + i * 1024), 16,
                                             xoff[i & 3] + (uint32_t)(i >> 2) * 16 * xrow_bytes,
                                             (uint32_t)g * kGroup * 2, 0, 0);
  };
  auto issue_x_all = [&](int g, int stage) {
#pragma unroll
    for (int i = 0; i < 16; ++i) issue_x_one(g, stage, i);
  };

  // Packed chunks and scales of this lane's columns.
  uint32_t woff[CB], soffs[CB];
#pragma unroll
  for (int cb = 0; cb < CB; ++cb) {
    const uint32_t nl = (uint32_t)(wave * WN + cb * 16 + lr);
    woff[cb] = nl * row_bytes + (uint32_t)lq * 4 * B;
    soffs[cb] = nl * (uint32_t)G * 4;
  }
  auto load_w = [&](int g, uint32_t (&w)[CB][B], float (&sc)[CB]) {
#pragma unroll
    for (int cb = 0; cb < CB; ++cb) {
      load_chunk_buf<B>(rw, woff[cb], (uint32_t)g * 16 * B, w[cb]);
      sc[cb] = __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(rs, soffs[cb],
                                                                            (uint32_t)g * 4, 0));
    }
  };

  // A operand of step u (sub-step u/16, row block u%16) from an LDS stage.
  uint32_t aoff[4];
#pragma unroll
  for (int s = 0; s < 4; ++s) aoff[s] = (uint32_t)(lr * 256 + (((4 * lq + s) ^ lr) * 16));
  auto read_a = [&](int stage, int u) -> bf16x8 {
    return *reinterpret_cast<const bf16x8*>(lds + stage * kLdsStage + (u & 15) * 4096 +
                                            aoff[u >> 4]);
  };

  f32x4 acc[RB][CB];
#pragma unroll
  for (int rb = 0; rb < RB; ++rb)
#pragma unroll
    for (int cb = 0; cb < CB; ++cb) acc[rb][cb] = f32x4{0.f, 0.f, 0.f, 0.f};

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
      for (int cb = 0; cb < CB; ++cb) {
        const int n = min(nw0 + wave * WN + cb * 16 + lr, args.n - 1);
        const bf16x8 v = *reinterpret_cast<const bf16x8*>(args.lora_up + (int64_t)n * R + kc);
        bl[cb] = kok ? v : zero;
      }
#pragma unroll
      for (int rb = 0; rb < RB; ++rb) {
        const int m = min(m0 + rb * 16 + lr, args.m - 1);
        const bf16x8 v = *reinterpret_cast<const bf16x8*>(args.t + (int64_t)m * R + kc);
        const bf16x8 al = kok ? v : zero;
#pragma unroll
        for (int cb = 0; cb < CB; ++cb) acc[rb][cb] = mfma16x16x32(al, bl[cb], acc[rb][cb]);
      }
    }
  }

  uint32_t wc[CB][B], wn[CB][B], be[CB][B];
  float sc[CB], sn[CB], ns64[CB];
  bf16x8 ring[RING];
  u32x4 bc[CB], bnx[CB];
  uint32_t nib[CB][2];                  // 4-bit: spread nibbles of the current dword

  auto take_next_weights = [&]() {
#pragma unroll
    for (int cb = 0; cb < CB; ++cb) {
#pragma unroll
      for (int j = 0; j < B; ++j) wc[cb][j] = wn[cb][j];
      sc[cb] = sn[cb];
      byteswap_chunk<B>(wc[cb], be[cb]);
      ns64[cb] = -64.0f * sc[cb];
    }
  };
  // dequantization job j of a sub-step: column block j / 4, bf16 pair j % 4
  auto dq_job = [&](int j, int S) {
    const int cb = j >> 2, p = j & 3;
    if constexpr (B == 4) {
      if (p == 0) spread_nibbles(wc[cb][S], nib[cb]);
    }
    bnx[cb][p] = dequant_pair<B>(be[cb], nib[cb], S, p, sc[cb], ns64[cb]);
  };

  // Group g uses LDS stage (g + G) % 2, so that after an optional lone first
  // group (odd G) the loop runs in (stage 0, stage 1) pairs.
  const int st0 = G & 1;
  issue_x_all(0, st0);
  load_w(0, wn, sn);
  __builtin_amdgcn_s_waitcnt(0);
  __syncthreads();
  take_next_weights();
#pragma unroll
  for (int u = 0; u < LA; ++u) ring[u % RING] = read_a(st0, u);
#pragma unroll
  for (int j = 0; j < 4 * CB; ++j) dq_job(j, 0);
#pragma unroll
  for (int cb = 0; cb < CB; ++cb) bc[cb] = bnx[cb];

  // One 128-group: 64 steps (4 sub-steps x 16 row blocks), CB MFMAs each.
  // Every step index is a compile-time constant (fold over an index sequence),
  // so the operand ring and the dequantization schedule are fully static:
  //   steps 0..15   one X DMA instruction each (next group -> idle stage)
  //   step 16       packed chunks + scales of the next group
  //   every step    one LDS read LA steps ahead, at most one dequantization
  //                 job (2 codes) for the next sub-step, CB MFMAs
  //   end of s = 2  switch to the next group's weights (their loads landed)
  //   step HAND     barrier: the next group's X is in LDS, this stage is free
  // The last group runs the same code: its "next group" is itself again
  // (clamped), fetched into the idle stage and never used.
  constexpr int JOBS = 4 * CB;
  auto group = [&](int g, auto stage_tag) {
    constexpr int ST = decltype(stage_tag)::value;
    const int gn = min(g + 1, G - 1);
    auto step = [&]<int T>(std::integral_constant<int, T>) {
      constexpr int s = T >> 4, rb = T & 15;
      if constexpr (T < 16) issue_x_one(gn, ST ^ 1, T);
      if constexpr (T == 16) load_w(gn, wn, sn);
      if constexpr (T == HAND) {
        __builtin_amdgcn_s_waitcnt(0);
        __syncthreads();
      }
      constexpr int u = T + LA;
      if constexpr (u < 64) {
        ring[u % RING] = read_a(ST, u);
      } else {
        ring[u % RING] = read_a(ST ^ 1, u - 64);
      }
      // jobs of the next sub-step (the next group's sub-step 0 during s = 3)
      [&]<int... J>(std::integer_sequence<int, J...>) {
        ([&] {
          if constexpr (J * 16 / JOBS == rb) dq_job(J, (s + 1) & 3);
        }(), ...);
      }(std::make_integer_sequence<int, JOBS>{});
      [&]<int... C>(std::integer_sequence<int, C...>) {
        ((acc[rb][C] = mfma16x16x32(ring[T % RING], __builtin_bit_cast(bf16x8, bc[C]),
                                    acc[rb][C])), ...);
      }(std::make_integer_sequence<int, CB>{});
      if constexpr (rb == 15) {
#pragma unroll
        for (int cb = 0; cb < CB; ++cb) bc[cb] = bnx[cb];
        if constexpr (s == 2) take_next_weights();
      }
      // interleave: MFMA, a few VALU, MFMA, ... (one wave per SIMD: the
      // dequantization must ride in the shadow of the matrix pipe)
#pragma unroll
      for (int cb = 0; cb < CB; ++cb) {
        __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
        __builtin_amdgcn_sched_group_barrier(0x002, 3, 0);
      }
      __builtin_amdgcn_sched_barrier(0);
    };
    [&]<int... T>(std::integer_sequence<int, T...>) {
      (step(std::integral_constant<int, T>{}), ...);
    }(std::make_integer_sequence<int, 64>{});
  };

  using I0 = std::integral_constant<int, 0>;
  using I1 = std::integral_constant<int, 1>;
  int g = 0;
  if (st0 == 1) group(g++, I1{});
  for (; g < G; g += 2) {
    group(g, I0{});
    group(g + 1, I1{});
  }

  const int ncol0 = nw0 + wave * WN;
  if (args.out_bf16) {
#pragma unroll
    for (int rb = 0; rb < RB; ++rb)
#pragma unroll
      for (int cb = 0; cb < CB; ++cb)
        store_tile<true>(args.y, args.n, m0 + rb * 16 + 4 * lq, ncol0 + cb * 16 + lr, args.m,
                         args.n, acc[rb][cb]);
  } else {
#pragma unroll
    for (int rb = 0; rb < RB; ++rb)
#pragma unroll
      for (int cb = 0; cb < CB; ++cb)
        store_tile<false>(args.y, args.n, m0 + rb * 16 + 4 * lq, ncol0 + cb * 16 + lr, args.m,
                          args.n, acc[rb][cb]);
  }
}

// ---------------------------------------------------------------------------
// K3: small-M GEMM (M <= 16*RB <= 64).  Workgroup = NW waves; it owns CB
// column blocks (16*CB columns) and the whole K range; wave w takes the
// groups g = w, w + NW, ...  Per group each lane loads its X row slice (the
// A operands, reused across the CB column blocks) and, per column block, its
// packed chunk + scale.  The NW partial tiles are summed through LDS.
// ---------------------------------------------------------------------------
template <int B, int RB, int CB, int NW>
__global__ __launch_bounds__(64 * NW) void gemm_small_kernel(GemmArgs args) {
  __shared__ f32x4 red[NW][RB * CB][64];
  const int wave = threadIdx.x >> 6;
  const int lane = threadIdx.x & 63;
  const int lr = lane & 15, lq = lane >> 4;
  const int n0 = blockIdx.x * 16 * CB;
  const int K = args.k;
  const int G = K / kGroup;
  const int64_t row_bytes = (int64_t)K * B / 8;

  const uint8_t* wptr[CB];
  const float* sptr[CB];
#pragma unroll
  for (int cb = 0; cb < CB; ++cb) {
    const int n = min(n0 + cb * 16 + lr, args.n - 1);
    wptr[cb] = args.packed + (int64_t)n * row_bytes + lq * 4 * B;
    sptr[cb] = args.scales + (int64_t)n * G;
  }
  const __bf16* xptr[RB];
  bool xok[RB];
#pragma unroll
  for (int rb = 0; rb < RB; ++rb) {
    const int m = rb * 16 + lr;
    xok[rb] = m < args.m;
    xptr[rb] = args.x + (int64_t)min(m, args.m - 1) * K + 32 * lq;
  }

  f32x4 acc[RB][CB];
#pragma unroll
  for (int rb = 0; rb < RB; ++rb)
#pragma unroll
    for (int cb = 0; cb < CB; ++cb) acc[rb][cb] = f32x4{0.f, 0.f, 0.f, 0.f};

  for (int g = wave; g < G; g += NW) {
    bf16x8 a[RB][4];
#pragma unroll
    for (int rb = 0; rb < RB; ++rb)
#pragma unroll
      for (int s = 0; s < 4; ++s)
        a[rb][s] = load_bf16x8_or_zero(xptr[rb] + g * kGroup + 8 * s, xok[rb]);
    uint32_t raw[CB][B], be[CB][B];
    float sc[CB], ns64[CB];
#pragma unroll
    for (int cb = 0; cb < CB; ++cb) {
      load_chunk<B>(wptr[cb] + (int64_t)g * 16 * B, raw[cb]);
      sc[cb] = sptr[cb][g];
    }
#pragma unroll
    for (int cb = 0; cb < CB; ++cb) {
      byteswap_chunk<B>(raw[cb], be[cb]);
      ns64[cb] = -64.0f * sc[cb];
      const bf16x8 b0 = dequant8<B>(raw[cb], be[cb], 0, sc[cb], ns64[cb]);
      const bf16x8 b1 = dequant8<B>(raw[cb], be[cb], 1, sc[cb], ns64[cb]);
      const bf16x8 b2 = dequant8<B>(raw[cb], be[cb], 2, sc[cb], ns64[cb]);
      const bf16x8 b3 = dequant8<B>(raw[cb], be[cb], 3, sc[cb], ns64[cb]);
#pragma unroll
      for (int rb = 0; rb < RB; ++rb) {
        acc[rb][cb] = mfma16x16x32(a[rb][0], b0, acc[rb][cb]);
        acc[rb][cb] = mfma16x16x32(a[rb][1], b1, acc[rb][cb]);
        acc[rb][cb] = mfma16x16x32(a[rb][2], b2, acc[rb][cb]);
        acc[rb][cb] = mfma16x16x32(a[rb][3], b3, acc[rb][cb]);
      }
    }
  }

  if (args.t != nullptr) {
    if (wave == 0) {
      const int R = args.r;
      for (int j0 = 0; j0 < R; j0 += 32) {
        const int kk = j0 + 8 * lq;
        const bool kok = kk < R;
#pragma unroll
        for (int cb = 0; cb < CB; ++cb) {
          const int n = min(n0 + cb * 16 + lr, args.n - 1);
          const bf16x8 bl = load_bf16x8_or_zero(args.lora_up + (int64_t)n * R + kk, kok);
#pragma unroll
          for (int rb = 0; rb < RB; ++rb) {
            const int m = min(rb * 16 + lr, args.m - 1);
            const bf16x8 al = load_bf16x8_or_zero(args.t + (int64_t)m * R + kk, kok);
            acc[rb][cb] = mfma16x16x32(al, bl, acc[rb][cb]);
          }
        }
      }
    }
  }

#pragma unroll
  for (int rb = 0; rb < RB; ++rb)
#pragma unroll
    for (int cb = 0; cb < CB; ++cb) red[wave][rb * CB + cb][lane] = acc[rb][cb];
  __syncthreads();
  // Sum the NW partial tiles; thread t handles tile entries t, t + 64*NW, ...
  for (int e = threadIdx.x; e < RB * CB * 64; e += 64 * NW) {
    const int tile = e / 64, ln = e % 64;
    f32x4 s = red[0][tile][ln];
#pragma unroll
    for (int w = 1; w < NW; ++w) {
      const f32x4 v = red[w][tile][ln];
      s[0] += v[0]; s[1] += v[1]; s[2] += v[2]; s[3] += v[3];
    }
    const int rb = tile / CB, cb = tile % CB;
    if (args.out_bf16)
      store_tile<true>(args.y, args.n, rb * 16 + 4 * (ln >> 4), n0 + cb * 16 + (ln & 15),
                       args.m, args.n, s);
    else
      store_tile<false>(args.y, args.n, rb * 16 + 4 * (ln >> 4), n0 + cb * 16 + (ln & 15),
                        args.m, args.n, s);
  }
}

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
