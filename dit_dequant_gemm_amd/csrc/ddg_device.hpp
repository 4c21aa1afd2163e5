// Device-side building blocks for the gfx950 kernels of libddg.
//
// Packed-code unpacking and dequantization (the Wan-Dancer-14B quantization
// report, §3.3 packed layout and §3.4 dequantize):
//   w_hat = bf16_rne(fl32((q_u - n_half) * scale)).
//
// A "chunk" is 32 consecutive codes of one row inside one 128-group.  With
// the MSB-first bitstream a chunk occupies exactly `B` dwords and starts on a
// dword boundary, for every bit width B in 3..7.  The GEMM kernels give each
// lane one chunk per (column, group) so that all 32 codes share one scale.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include <utility>

namespace ddg {

typedef __bf16 bf16x8 __attribute__((__vector_size__(8 * sizeof(__bf16))));
typedef __bf16 bf16x2 __attribute__((__vector_size__(2 * sizeof(__bf16))));
typedef float f32x4 __attribute__((__vector_size__(4 * sizeof(float))));
typedef float f32x16 __attribute__((__vector_size__(16 * sizeof(float))));
typedef uint32_t u32x4 __attribute__((__vector_size__(4 * sizeof(uint32_t))));
typedef uint32_t u32x2 __attribute__((__vector_size__(2 * sizeof(uint32_t))));

constexpr int kGroup = 128;

template <int B>
struct Bits {
  static constexpr int n_half = (1 << (B - 1)) - 1;     // largest |q|
  static constexpr uint32_t mask = (1u << B) - 1;
  // q + 64 = q_u + (64 - n_half): a byte in [1, 127] for every B <= 7, so that
  // fma(q + 64, s, -64 s) = fl32(q * s) with one rounding (64 s is exact).
  static constexpr uint32_t bias64 = 64u - (uint32_t)n_half;
};

// Two floats -> packed bf16 pair (round to nearest even; v_cvt_pk_bf16_f32).
__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
  bf16x2 v = {(__bf16)lo, (__bf16)hi};
  return __builtin_bit_cast(uint32_t, v);
}

// Bytes 2H, 2H+1 of w as floats, for bytes below 16 (codes plus one): an E4M3
// byte whose top nibble is zero has exponent field 0 (value m 2^-9) or 1
// (value (8 + m) 2^-9), i.e. the byte's integer value times 2^-9, so the
// scaled FP8 conversion with scale 2^9 returns the integer exactly, two
// bytes per instruction (v_cvt_scalef32_pk_f32_fp8).
typedef float f32x2 __attribute__((ext_vector_type(2)));
template <int H>
__device__ __forceinline__ f32x2 small_bytes_f32(uint32_t w) {
  return __builtin_amdgcn_cvt_scalef32_pk_f32_fp8(w, 512.0f, H != 0);
}

// fl32(q * s) given v = q + 64 as a float and ns64 = -64 * s.
__device__ __forceinline__ float scale_code(float v, float s, float ns64) {
  return __builtin_fmaf(v, s, ns64);
}

// Code I (0..31) of a chunk whose dwords were byte-swapped into `be`
// (big-endian words: stream bit 32*j is the MSB of be[j]).
template <int B>
__device__ __forceinline__ uint32_t chunk_code(const uint32_t* be, int i) {
  const int o = i * B, j = o >> 5, off = o & 31;
  if (off + B <= 32) return (be[j] >> (32 - off - B)) & Bits<B>::mask;
  return __builtin_amdgcn_alignbit(be[j], be[j + 1], 64 - off - B) & Bits<B>::mask;
}

// Dequantize codes 8*S .. 8*S+7 of a chunk into one MFMA operand (8 bf16,
// element e = code 8*S+e).  `raw` holds the chunk's dwords as loaded
// (little-endian), `be` the same dwords byte-swapped (unused for B == 4).
// S must fold to a constant after inlining and unrolling.
template <int B>
__device__ __forceinline__ bf16x8 dequant8(const uint32_t* raw, const uint32_t* be, int S,
                                           float s, float ns64) {
  u32x4 out;
  if constexpr (B == 4) {
    // Dword S holds codes 8S..8S+7; byte p holds code 8S+2p in its high
    // nibble and 8S+2p+1 in its low nibble.
    const uint32_t x = raw[S];
    const uint32_t ev = ((x >> 4) & 0x0F0F0F0Fu) + 0x01010101u * Bits<4>::bias64;
    const uint32_t od = (x & 0x0F0F0F0Fu) + 0x01010101u * Bits<4>::bias64;
#pragma unroll
    for (int p = 0; p < 4; ++p) {
      const float a = (float)((ev >> (8 * p)) & 0xFFu);
      const float b = (float)((od >> (8 * p)) & 0xFFu);
      out[p] = pack_bf16x2(scale_code(a, s, ns64), scale_code(b, s, ns64));
    }
  } else {
#pragma unroll
    for (int p = 0; p < 4; ++p) {
      const uint32_t c0 = chunk_code<B>(be, 8 * S + 2 * p) + Bits<B>::bias64;
      const uint32_t c1 = chunk_code<B>(be, 8 * S + 2 * p + 1) + Bits<B>::bias64;
      out[p] = pack_bf16x2(scale_code((float)c0, s, ns64), scale_code((float)c1, s, ns64));
    }
  }
  return __builtin_bit_cast(bf16x8, out);
}

// Pair P (codes 8*S+2P, 8*S+2P+1) of a chunk as one packed bf16 pair.  For
// B == 4, `nib` holds the two words of spread_nibbles for dword S (codes plus
// one, as bytes) and nb = -8 s; otherwise `be` holds the byte-swapped dwords
// and nb = -64 s (codes plus 64).  S and P must fold to constants after
// inlining.
template <int B>
__device__ __forceinline__ uint32_t dequant_pair(const uint32_t* be, const uint32_t* nib, int S,
                                                 int P, float s, float nb) {
  if constexpr (B == 4) {
    const f32x2 e = (P >> 1) ? small_bytes_f32<1>(nib[0]) : small_bytes_f32<0>(nib[0]);
    const f32x2 o = (P >> 1) ? small_bytes_f32<1>(nib[1]) : small_bytes_f32<0>(nib[1]);
    return pack_bf16x2(__builtin_fmaf((P & 1) ? e.y : e.x, s, nb),
                       __builtin_fmaf((P & 1) ? o.y : o.x, s, nb));
  } else {
    const uint32_t c0 = chunk_code<B>(be, 8 * S + 2 * P) + Bits<B>::bias64;
    const uint32_t c1 = chunk_code<B>(be, 8 * S + 2 * P + 1) + Bits<B>::bias64;
    return pack_bf16x2(scale_code((float)c0, s, nb), scale_code((float)c1, s, nb));
  }
}

// ---------------------------------------------------------------------------
// "Plus-one" form, used by the M <= 16 kernel.  Every code q_u is at most
// 2^B - 2, so q_u + 1 still fits its B-bit field: one 32-bit add of a
// constant with a 1 at the lowest bit of every field that lies wholly in a
// word adds 1 to all of them at once, with no carry between fields.  Then
// fl32((q_u - n_half) * s) = fma(q_u + 1, s, -2^(B-1) s), the constant being
// exact (a power-of-two multiple of s), so the product is rounded once.
// ---------------------------------------------------------------------------
template <int B>
struct PlusOne {
  // the add constant for big-endian word j of a 32-code chunk
  static constexpr uint32_t word_add(int j) {
    uint32_t a = 0;
    for (int c = 0; c < 32; ++c) {
      const int o = c * B - 32 * j;
      if (o >= 0 && o + B <= 32) a |= 1u << (32 - o - B);
    }
    return a;
  }
};

// Byte-swapped chunk words with 1 added to every whole field (B != 4).
template <int B>
__device__ __forceinline__ void plus_one_words(const uint32_t* raw, uint32_t* be1) {
  [&]<int... J>(std::integer_sequence<int, J...>) {
    ((be1[J] = __builtin_bswap32(raw[J]) + PlusOne<B>::word_add(J)), ...);
  }(std::make_integer_sequence<int, B>{});
}

// Code I of the chunk plus one, from plus_one_words output.
template <int B>
__device__ __forceinline__ uint32_t chunk_code_p1(const uint32_t* be1, int i) {
  const int o = i * B, j = o >> 5, off = o & 31;
  if (off + B <= 32) return (be1[j] >> (32 - off - B)) & Bits<B>::mask;
  // a field across two words was not incremented by the word adds
  return (__builtin_amdgcn_alignbit(be1[j], be1[j + 1], 64 - off - B) & Bits<B>::mask) + 1u;
}

// Codes 8S .. 8S+7 of a chunk as one MFMA operand, plus-one form.  For
// B == 4, x1 = dword S of the chunk plus 0x11111111 (byte p holds codes
// 8S+2p, 8S+2p+1 in its high, low nibble); otherwise be1 from plus_one_words.
// nsh = -2^(B-1) * s.  S must fold to a constant.
template <int B>
__device__ __forceinline__ bf16x8 dequant8_p1(const uint32_t* be1, uint32_t x1, int S, float s,
                                              float nsh) {
  u32x4 out;
  if constexpr (B == 4) {
    uint32_t ev = (x1 >> 4) & 0x0F0F0F0Fu;
    uint32_t od = x1 & 0x0F0F0F0Fu;
    // keep the two masked words: two bytes then convert per instruction
    asm("" : "+v"(ev), "+v"(od));
    const f32x2 e0 = small_bytes_f32<0>(ev), e1 = small_bytes_f32<1>(ev);
    const f32x2 o0 = small_bytes_f32<0>(od), o1 = small_bytes_f32<1>(od);
    out[0] = pack_bf16x2(__builtin_fmaf(e0.x, s, nsh), __builtin_fmaf(o0.x, s, nsh));
    out[1] = pack_bf16x2(__builtin_fmaf(e0.y, s, nsh), __builtin_fmaf(o0.y, s, nsh));
    out[2] = pack_bf16x2(__builtin_fmaf(e1.x, s, nsh), __builtin_fmaf(o1.x, s, nsh));
    out[3] = pack_bf16x2(__builtin_fmaf(e1.y, s, nsh), __builtin_fmaf(o1.y, s, nsh));
  } else {
#pragma unroll
    for (int p = 0; p < 4; ++p) {
      const float a = (float)chunk_code_p1<B>(be1, 8 * S + 2 * p);
      const float b = (float)chunk_code_p1<B>(be1, 8 * S + 2 * p + 1);
      out[p] = pack_bf16x2(__builtin_fmaf(a, s, nsh), __builtin_fmaf(b, s, nsh));
    }
  }
  return __builtin_bit_cast(bf16x8, out);
}

// 4-bit only: dword x -> {even codes, odd codes} plus one, as bytes (every
// code is at most 14, so adding 1 to each nibble carries into no other).
__device__ __forceinline__ void spread_nibbles(uint32_t x, uint32_t* nib) {
  const uint32_t x1 = x + 0x11111111u;
  nib[0] = (x1 >> 4) & 0x0F0F0F0Fu;
  nib[1] = x1 & 0x0F0F0F0Fu;
}

template <int B>
__device__ __forceinline__ void byteswap_chunk(const uint32_t* raw, uint32_t* be) {
  if constexpr (B != 4) {
#pragma unroll
    for (int j = 0; j < B; ++j) be[j] = __builtin_bswap32(raw[j]);
  }
}

// Load the B dwords of one chunk (4-byte aligned; 16-byte aligned for B == 4).
template <int B>
__device__ __forceinline__ void load_chunk(const uint8_t* p, uint32_t* raw) {
  if constexpr (B == 4) {
    const u32x4 v = *reinterpret_cast<const u32x4*>(p);
    raw[0] = v[0]; raw[1] = v[1]; raw[2] = v[2]; raw[3] = v[3];
  } else if constexpr (B == 6) {
    const u32x2* q = reinterpret_cast<const u32x2*>(p);   // chunk offsets are 8-byte aligned
#pragma unroll
    for (int j = 0; j < 3; ++j) { const u32x2 v = q[j]; raw[2 * j] = v[0]; raw[2 * j + 1] = v[1]; }
  } else {
    const uint32_t* q = reinterpret_cast<const uint32_t*>(p);
#pragma unroll
    for (int j = 0; j < B; ++j) raw[j] = q[j];
  }
}

// Buffer resources (gfx9 family descriptor word 3).  Loads past num_records
// return zeros, so tiles that hang over the M or N edge need no clamping.
constexpr int kBufferFlags = 0x00020000;
typedef __amdgpu_buffer_rsrc_t rsrc_t;
typedef __attribute__((address_space(3))) void* lds_ptr_t;

__device__ __forceinline__ rsrc_t make_rsrc(const void* base, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, (int)bytes,
                                           kBufferFlags);
}

// x / s correctly rounded without a division, by Markstein's correction
// (P. Markstein, "Computation of elementary functions on the IBM RISC
// System/6000 processor", 1990): if y = RN(1/s) and q is within an ulp of
// x / s, then with the residual r = x - q s (exact through the FMA),
// RN(q + r y) = RN(x / s), barring over- and underflow.  One correction
// brings the plain product RN(x y) within half an ulp (plus a term of
// relative size 2^-24), the second one then rounds correctly.  The callers
// use it for scales in [2^-60, 2^100] and |x / s| at most the format's
// largest value: for |x| >= 2^-96 the residual stays a normal number, and
// smaller x give quotients below 2^-36, code 0 in every format here.
// (Checked against exact rational division on 144,000 bf16 x and random s.)
__device__ __forceinline__ float div_markstein(float x, float s, float y) {
  float q = x * y;
  float r = __builtin_fmaf(-q, s, x);
  q = __builtin_fmaf(r, y, q);
  r = __builtin_fmaf(-q, s, x);
  return __builtin_fmaf(r, y, q);
}
__device__ __forceinline__ bool markstein_ok(float s) { return s >= 0x1p-60f && s <= 0x1p100f; }

// v[i] / s for N values in place (0 for a zero scale): the correction above
// when the scale allows it, else the IEEE division; one branch for all N so
// that the division code is skipped when no lane needs it.
template <int N>
__device__ __forceinline__ void quotients(float (&v)[N], bool zero, bool fast, float s, float y) {
  if (zero) {
#pragma unroll
    for (int i = 0; i < N; ++i) v[i] = 0.0f;
  } else if (fast) {
#pragma unroll
    for (int i = 0; i < N; ++i) v[i] = div_markstein(v[i], s, y);
  } else {
#pragma unroll
    for (int i = 0; i < N; ++i) v[i] = v[i] / s;
  }
}

// Epilogue store of one 32 x 32 fp32 block held in the 32x32 MFMA output
// layout (lane: column lane % 32, rows 8 (r / 4) + 4 (lane / 32) + r % 4,
// r = 0..15) into row-major Y (m x n, bf16 or fp32).  The block goes through
// a per-wave LDS scratch (32 rows x 40 floats: the 8-float pad puts the two
// lane halves' rows, 4 apart, on different banks) and leaves as 16-byte
// pieces of rows: 2 (bf16) or 4 (fp32) stores per lane instead of 16 two-
// or four-byte ones.  Rows >= m and columns >= n are not written.  vec: n
// and y allow 16-byte stores (n a multiple of 8 for bf16, 4 for fp32, y
// 16-byte aligned); otherwise element stores.  bf16 is the round to nearest
// even of the fp32 value, as a direct store.  The scratch belongs to the
// calling wave alone; LDS serves one wave's accesses in order, so the reads
// see the writes once lgkmcnt is 0.
constexpr int kEpiStride = 40;
constexpr int kEpiScratch = 32 * kEpiStride * 4;          // bytes per wave

// 16 aligned bytes of a product's output, written through the L2 (cache
// policy SC1).  When a kernel ends, the dirty lines in the 8 XCDs' L2s are
// written back before the next kernel on the stream starts; output already
// written through leaves less to write back.  Back-to-back
// 4096 x 3072 x 3072 products on 256 x 192 tiles went from 73.7 to 70.2 us
// per launch; on 256 x 256 tiles, 32760 x 5120 x 5120 and 4096 x 12288 x 3072
// stayed within 1%.  The store is written in assembly because the global-store
// builtins take no cache-policy operand.  Pairs of 8-byte agent-scope atomic
// stores do compile to SC1 stores, but they made the large products 4-5%
// slower.  The s_nop after the store covers the hazard of a vector ALU
// instruction writing the data registers of a store of more than 8 bytes
// right after it.  The compiler does not count this store in its memory
// waits.  Vector memory operations complete in issue order, so that only
// makes its waits for later loads stricter.
__device__ __forceinline__ void store_out16(void* p, u32x4 v) {
  asm volatile("global_store_dwordx4 %0, %1, off sc1\n\ts_nop 1" : : "v"(p), "v"(v) : "memory");
}

template <bool BF16, typename V>
__device__ __forceinline__ void store_block32(const V& v, float* scratch, void* y, int m, int n, int row0,
                                              int col0, bool vec) {
  const int lane = threadIdx.x & 63, lr = lane & 31, lh = lane >> 5;
#pragma unroll
  for (int r = 0; r < 16; ++r) scratch[(8 * (r >> 2) + 4 * lh + (r & 3)) * kEpiStride + lr] = v[r];
  __builtin_amdgcn_s_waitcnt(0xC07F);                      // lgkmcnt(0)
  __builtin_amdgcn_wave_barrier();
  constexpr int W = BF16 ? 8 : 4;                          // values per 16-byte piece
  constexpr int PER_ROW = 32 / W;
  // a block wholly inside Y with 16-byte-aligned rows: no per-lane checks
  // (one uniform branch instead of a divergent one per piece)
  if (vec && row0 + 32 <= m && col0 + 32 <= n) {
#pragma unroll
    for (int i = 0; i < 32 * PER_ROW / 64; ++i) {
      const int q = lane + 64 * i;
      const int row = q / PER_ROW, c = (q % PER_ROW) * W;
      float f[W];
#pragma unroll
      for (int j = 0; j < W / 4; ++j) {
        const f32x4 t = *reinterpret_cast<const f32x4*>(scratch + row * kEpiStride + c + 4 * j);
        f[4 * j] = t[0]; f[4 * j + 1] = t[1]; f[4 * j + 2] = t[2]; f[4 * j + 3] = t[3];
      }
      const int64_t base = (int64_t)(row0 + row) * n + col0 + c;
      if constexpr (BF16) {
        __bf16 b[8];
#pragma unroll
        for (int e = 0; e < 8; ++e) b[e] = (__bf16)f[e];
        store_out16(static_cast<__bf16*>(y) + base, __builtin_bit_cast(u32x4, b));
      } else {
        f32x4 t = {f[0], f[1], f[2], f[3]};
        store_out16(static_cast<float*>(y) + base, __builtin_bit_cast(u32x4, t));
      }
    }
    __builtin_amdgcn_wave_barrier();
    return;
  }
#pragma unroll
  for (int i = 0; i < 32 * PER_ROW / 64; ++i) {
    const int q = lane + 64 * i;
    const int row = q / PER_ROW, c = (q % PER_ROW) * W;
    float f[W];
#pragma unroll
    for (int j = 0; j < W / 4; ++j) {
      const f32x4 t = *reinterpret_cast<const f32x4*>(scratch + row * kEpiStride + c + 4 * j);
      f[4 * j] = t[0]; f[4 * j + 1] = t[1]; f[4 * j + 2] = t[2]; f[4 * j + 3] = t[3];
    }
    const int gr = row0 + row, gc = col0 + c;
    if (gr < m) {
      const int64_t base = (int64_t)gr * n + gc;
      if (vec && gc + W <= n) {
        if constexpr (BF16) {
          __bf16 b[8];
#pragma unroll
          for (int e = 0; e < 8; ++e) b[e] = (__bf16)f[e];
          store_out16(static_cast<__bf16*>(y) + base, __builtin_bit_cast(u32x4, b));
        } else {
          f32x4 t = {f[0], f[1], f[2], f[3]};
          store_out16(static_cast<float*>(y) + base, __builtin_bit_cast(u32x4, t));
        }
      } else {
#pragma unroll
        for (int e = 0; e < W; ++e) {
          if (gc + e < n) {
            if constexpr (BF16)
              static_cast<__bf16*>(y)[base + e] = (__bf16)f[e];
            else
              static_cast<float*>(y)[base + e] = f[e];
          }
        }
      }
    }
  }
  __builtin_amdgcn_wave_barrier();
}

// 16-byte stores are possible for every row of an m x n output at y.
__device__ __forceinline__ bool epi_vec_ok(const void* y, int n, bool bf16) {
  return ((reinterpret_cast<uintptr_t>(y) & 15) == 0) && (n % (bf16 ? 8 : 4) == 0);
}

// Workgroup barrier that orders LDS only (waits on lgkmcnt, not vmcnt):
// global loads and stores stay in flight across it.
__device__ __forceinline__ void lds_barrier() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup", "local");
  __builtin_amdgcn_s_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup", "local");
}

// The B dwords of one chunk through a buffer resource (dword-aligned offsets).
template <int B>
__device__ __forceinline__ void load_chunk_buf(rsrc_t r, uint32_t voff, uint32_t soff,
                                               uint32_t* raw) {
  typedef uint32_t v4 __attribute__((ext_vector_type(4)));
  typedef uint32_t v3 __attribute__((ext_vector_type(3)));
  typedef uint32_t v2 __attribute__((ext_vector_type(2)));
  if constexpr (B == 3) {
    const v3 a = __builtin_amdgcn_raw_buffer_load_b96(r, voff, soff, 0);
    raw[0] = a.x; raw[1] = a.y; raw[2] = a.z;
  } else {
    const v4 a = __builtin_amdgcn_raw_buffer_load_b128(r, voff, soff, 0);
    raw[0] = a.x; raw[1] = a.y; raw[2] = a.z; raw[3] = a.w;
    if constexpr (B == 5) {
      raw[4] = __builtin_amdgcn_raw_buffer_load_b32(r, voff + 16, soff, 0);
    } else if constexpr (B == 6) {
      const v2 b = __builtin_amdgcn_raw_buffer_load_b64(r, voff + 16, soff, 0);
      raw[4] = b.x; raw[5] = b.y;
    } else if constexpr (B == 7) {
      const v3 b = __builtin_amdgcn_raw_buffer_load_b96(r, voff + 16, soff, 0);
      raw[4] = b.x; raw[5] = b.y; raw[6] = b.z;
    }
  }
}

__device__ __forceinline__ f32x4 mfma16x16x32(bf16x8 a, bf16x8 b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}

__device__ __forceinline__ float bf16_bits_to_f32(uint32_t h) {
  return __builtin_bit_cast(float, h << 16);
}

}  // namespace ddg
