// FP4 weights x FP8 or FP6 activations (W4A8, W4A6) on the gfx950 scaled
// matrix instructions (the FP4DiT article: 4-bit floating-point weight
// formats in groups of 128, §3.2.1 / §4.1; 8- and 6-bit per-token
// activations, §3.2.3 / §4.1):
//   fp4_quantize_pack_kernel  per-group(128) scale + nearest 4-bit level, packed
//                             two codes per byte (even index in the low nibble)
//   fp8_quantize_rows_kernel  per-token scale + E4M3 round-to-nearest-even
//   fp6_quantize_rows_kernel  per-token scale + E2M3 / E3M2 rounding, written
//                             in the tiled 6-bit storage the product reads
//   w4a8_gemm_kernel          Y = s_x[m] sum_g s_w[n,g] (X_q W_q^T)_g
#include "ddg_launch.hpp"

namespace ddg {

namespace {

// Magnitudes by index, and the midpoints between neighbours (exact in float32).
//   E2M1: 0 .5 1 1.5 2 3 4 6    E3M0: 0 .25 .5 1 2 4 8 16    E1M2: 0 .25 .. 1.75
template <int FMT>
struct Fp4Fmt;
template <>
struct Fp4Fmt<kFp4E2M1> {
  static constexpr float vmax = 6.0f;
  static constexpr float mid[7] = {0.25f, 0.75f, 1.25f, 1.75f, 2.5f, 3.5f, 5.0f};
};
template <>
struct Fp4Fmt<kFp4E3M0> {
  static constexpr float vmax = 16.0f;
  static constexpr float mid[7] = {0.125f, 0.375f, 0.75f, 1.5f, 3.0f, 6.0f, 12.0f};
};
template <>
struct Fp4Fmt<kFp4E1M2> {
  static constexpr float vmax = 1.75f;
  static constexpr float mid[7] = {0.125f, 0.375f, 0.625f, 0.875f, 1.125f, 1.375f, 1.625f};
};

// E4M3 bytes of the 8 magnitudes of each 4-bit format (all exact in E4M3),
// as two little-endian words: magnitudes 0-3, 4-7.
template <int FMT>
struct Fp4AsE4M3;
template <>
struct Fp4AsE4M3<kFp4E2M1> {   // 0 .5 1 1.5 | 2 3 4 6
  static constexpr uint32_t lo = 0x3C383000u, hi = 0x4C484440u;
};
template <>
struct Fp4AsE4M3<kFp4E3M0> {   // 0 .25 .5 1 | 2 4 8 16
  static constexpr uint32_t lo = 0x38302800u, hi = 0x58504840u;
};
template <>
struct Fp4AsE4M3<kFp4E1M2> {   // 0 .25 .5 .75 | 1 1.25 1.5 1.75
  static constexpr uint32_t lo = 0x34302800u, hi = 0x3E3C3A38u;
};

// Eight 4-bit codes (code i in bits 4i) -> eight E4M3 bytes in code order.
template <int FMT>
__device__ __forceinline__ u32x2 fp4_codes_to_e4m3(uint32_t x) {
  const uint32_t ev = x & 0x0F0F0F0Fu;                 // codes 0 2 4 6, one per byte
  const uint32_t od = (x >> 4) & 0x0F0F0F0Fu;          // codes 1 3 5 7
  auto conv = [](uint32_t c) {
    const uint32_t mag = __builtin_amdgcn_perm(Fp4AsE4M3<FMT>::hi, Fp4AsE4M3<FMT>::lo, c & 0x07070707u);
    return mag | ((c & 0x08080808u) << 4);
  };
  const uint32_t e = conv(ev), o = conv(od);
  u32x2 r;
  r[0] = __builtin_amdgcn_perm(o, e, 0x05010400u);    // e0 o0 e1 o1
  r[1] = __builtin_amdgcn_perm(o, e, 0x07030602u);    // e2 o2 e3 o3
  return r;
}

// Index of the level nearest a (>= 0): count the midpoints below it; on a
// midpoint move up only to an even index.
template <int FMT>
__device__ __forceinline__ uint32_t fp4_index(float a) {
  uint32_t idx = 0;
#pragma unroll
  for (int j = 0; j < 7; ++j) {
    const float mj = Fp4Fmt<FMT>::mid[j];
    idx += (a > mj || (a == mj && ((j + 1) & 1) == 0)) ? 1u : 0u;
  }
  return idx;
}

// The smallest power of two >= s (s >= 0 finite; 0 stays 0), at least 2^-126:
// the block-scale form (E8M0) the matrix instructions apply themselves.
__device__ __forceinline__ float pow2_at_least(float s) {
  const uint32_t b = __builtin_bit_cast(uint32_t, s);
  const uint32_t e = b & 0x7F800000u;
  uint32_t r;
  if (b == 0u) r = 0u;
  else if (e == 0u) r = 0x00800000u;                  // below 2^-126
  else if ((b & 0x007FFFFFu) == 0u) r = b;            // already a power of two
  else r = e + 0x00800000u;
  return __builtin_bit_cast(float, r);
}

// One lane per 32 consecutive weights (chunk c: row c / cpr, chunk c % cpr
// of the row, cpr = k / 32); the four lanes of a 128-group share the abs-max
// through a quad butterfly.  Output: 4 dwords of codes per lane (code 8 j + i
// in bits 4 i of dword j) and one scale per group, in row order or tiled:
// 32-column blocks, each (block, group) 2048 bytes in the order the matrix
// operands load them (see w4a8_gemm_kernel), the last block padded with zero
// codes and scales (chunks n_in .. n_out - 1 read no input).
template <int FMT, bool F32_IN, bool POW2, bool TILED>
__global__ __launch_bounds__(256) void fp4_quantize_pack_kernel(const void* __restrict__ w,
                                                               int64_t n_in, int64_t n_out, int cpr,
                                                               uint32_t* __restrict__ packed,
                                                               float* __restrict__ scales) {
  const int64_t c = (int64_t)blockIdx.x * 256 + threadIdx.x;
  const bool valid = c < n_out;
  const bool has_src = c < n_in;
  const int64_t cc = has_src ? c : 0;
  float v[32];
  if (!has_src) {
#pragma unroll
    for (int i = 0; i < 32; ++i) v[i] = 0.0f;
  } else if constexpr (F32_IN) {
    const f32x4* src = reinterpret_cast<const f32x4*>(static_cast<const float*>(w) + cc * 32);
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const f32x4 t = src[i];
      v[4 * i] = t[0]; v[4 * i + 1] = t[1]; v[4 * i + 2] = t[2]; v[4 * i + 3] = t[3];
    }
  } else {
    const u32x4* src = reinterpret_cast<const u32x4*>(static_cast<const uint16_t*>(w) + cc * 32);
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
  float a = 0.0f;
#pragma unroll
  for (int i = 0; i < 32; ++i) a = __builtin_fmaxf(a, __builtin_fabsf(v[i]));
  a = __builtin_fmaxf(a, __shfl_xor(a, 1));
  a = __builtin_fmaxf(a, __shfl_xor(a, 2));
  float s = a / Fp4Fmt<FMT>::vmax;
  if constexpr (POW2) s = pow2_at_least(s);
  const bool zero = !(s != 0.0f);
  u32x4 out = {0u, 0u, 0u, 0u};
#pragma unroll
  for (int i = 0; i < 32; ++i) {
    const float r = zero ? 0.0f : v[i] / s;
    const uint32_t idx = fp4_index<FMT>(__builtin_fabsf(r));
    const uint32_t code = idx | ((r < 0.0f && idx != 0u) ? 8u : 0u);
    out[i >> 3] |= code << (4 * (i & 7));
  }
  if (valid) {
    if constexpr (TILED) {
      const int64_t row = c / cpr;
      const int j = (int)(c - row * cpr);
      const int64_t G = cpr / 4, g = j >> 2, q = j & 3;
      const int64_t blk = (row >> 5) * G + g, lr = row & 31;
      reinterpret_cast<u32x4*>(packed)[blk * 128 + (q >> 1) * 64 + (q & 1) * 32 + lr] = out;
      if (q == 0) scales[blk * 32 + lr] = zero ? 0.0f : s;
    } else {
      reinterpret_cast<u32x4*>(packed)[c] = out;
      if ((threadIdx.x & 3) == 0) scales[c >> 2] = zero ? 0.0f : s;
    }
  }
}

// E4M3 code of a finite float: clamp to +-448, round to nearest even
// (subnormals: multiples of 2^-9; normals: three mantissa bits).
__device__ __forceinline__ uint32_t e4m3_code(float r) {
  const float a = __builtin_fminf(__builtin_fabsf(r), 448.0f);
  uint32_t mag;
  if (a < 0.015625f) {
    mag = (uint32_t)__builtin_rintf(a * 512.0f);
  } else {
    uint32_t b = __builtin_bit_cast(uint32_t, a);
    b += 0x7FFFFu + ((b >> 20) & 1u);
    mag = ((((b >> 23) - 127u + 7u) & 15u) << 3) | ((b >> 20) & 7u);
  }
  return (mag != 0u && r < 0.0f) ? (mag | 0x80u) : mag;
}



// E4M3 codes of two floats of magnitude <= 448 through the conversion
// instruction (OCP E4M3, round to nearest even), into byte pair P of w; a
// value that rounds to zero gets code 0 (the instruction keeps the sign).
__device__ __forceinline__ uint32_t e4m3_zero_fix(uint32_t w) {
  const uint32_t mag = w & 0x7F7F7F7Fu;
  const uint32_t nz = ((mag + 0x7F7F7F7Fu) | mag) & 0x80808080u;     // bit 7 of a byte: magnitude != 0
  return w & (0x7F7F7F7Fu | nz);
}

// E4M3 codes of eight values (one 16-byte bf16 chunk), r = x / s correctly
// rounded (see div_markstein) and clamped to +-448.
__device__ __forceinline__ u32x2 e4m3_chunk(u32x4 t, bool zero, bool fast, float s, float y) {
  float r[8];
#pragma unroll
  for (int j = 0; j < 8; ++j) r[j] = bf16_bits_to_f32((j & 1) ? (t[j >> 1] >> 16) : (t[j >> 1] & 0xFFFFu));
  quotients<8>(r, zero, fast, s, y);
#pragma unroll
  for (int j = 0; j < 8; ++j) r[j] = __builtin_fminf(__builtin_fmaxf(r[j], -448.0f), 448.0f);
  u32x2 o;
#pragma unroll
  for (int w = 0; w < 2; ++w) {
    int p = __builtin_amdgcn_cvt_pk_fp8_f32(r[4 * w], r[4 * w + 1], 0, false);
    p = __builtin_amdgcn_cvt_pk_fp8_f32(r[4 * w + 2], r[4 * w + 3], p, true);
    o[w] = e4m3_zero_fix((uint32_t)p);
  }
  return o;
}

// One workgroup of 256 lanes per row for rows up to 2048 * NCH wide: lane i
// reads chunks i, i + 256, ... (at most NCH of them) once, keeps them in
// registers for the abs-max (wave butterfly, then the four waves through
// LDS) and converts them.
template <int NCH>
__global__ __launch_bounds__(256) void fp8_quantize_rows_reg_kernel(const uint16_t* __restrict__ x, int k,
                                                                   uint8_t* __restrict__ q,
                                                                   float* __restrict__ sx) {
  __shared__ float part[4];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int64_t row = blockIdx.x;
  const u32x4* src = reinterpret_cast<const u32x4*>(x + row * k);
  const int chunks = k / 8;
  u32x4 t[NCH];
  float a = 0.0f;
#pragma unroll
  for (int i = 0; i < NCH; ++i) {
    const int c = tid + 256 * i;
    t[i] = c < chunks ? src[c] : u32x4{0u, 0u, 0u, 0u};
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      a = __builtin_fmaxf(a, __builtin_fabsf(bf16_bits_to_f32(t[i][j] & 0xFFFFu)));
      a = __builtin_fmaxf(a, __builtin_fabsf(bf16_bits_to_f32(t[i][j] >> 16)));
    }
  }
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) a = __builtin_fmaxf(a, __shfl_xor(a, off));
  if (lane == 0) part[wave] = a;
  __syncthreads();
  a = __builtin_fmaxf(__builtin_fmaxf(part[0], part[1]), __builtin_fmaxf(part[2], part[3]));
  const float s = a / 448.0f;
  const bool zero = !(s != 0.0f);
  const bool fast = markstein_ok(s);
  const float y = fast ? 1.0f / s : 0.0f;
  u32x2* dst = reinterpret_cast<u32x2*>(q + row * k);
#pragma unroll
  for (int i = 0; i < NCH; ++i) {
    const int c = tid + 256 * i;
    if (c < chunks) dst[c] = e4m3_chunk(t[i], zero, fast, s, y);
  }
  if (tid == 0) sx[row] = zero ? 0.0f : s;
}

// Wider rows: one wave per row (four rows per workgroup), two passes over
// the row: the row's abs-max, then r = x / s and its E4M3 code, eight codes
// per lane and step.
__global__ __launch_bounds__(256) void fp8_quantize_rows_kernel(const uint16_t* __restrict__ x,
                                                               int64_t m, int k,
                                                               uint8_t* __restrict__ q,
                                                               float* __restrict__ sx) {
  const int lane = threadIdx.x & 63;
  const int64_t row = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
  if (row >= m) return;
  const u32x4* src = reinterpret_cast<const u32x4*>(x + row * k);
  const int chunks = k / 8;
  float a = 0.0f;
#pragma unroll 4
  for (int c = lane; c < chunks; c += 64) {
    const u32x4 t = src[c];
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      a = __builtin_fmaxf(a, __builtin_fabsf(bf16_bits_to_f32(t[j] & 0xFFFFu)));
      a = __builtin_fmaxf(a, __builtin_fabsf(bf16_bits_to_f32(t[j] >> 16)));
    }
  }
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) a = __builtin_fmaxf(a, __shfl_xor(a, off));
  const float s = a / 448.0f;
  const bool zero = !(s != 0.0f);
  const bool fast = markstein_ok(s);
  const float y = fast ? 1.0f / s : 0.0f;
  u32x2* dst = reinterpret_cast<u32x2*>(q + row * k);
#pragma unroll 4
  for (int c = lane; c < chunks; c += 64) dst[c] = e4m3_chunk(src[c], zero, fast, s, y);
  if (lane == 0) sx[row] = zero ? 0.0f : s;
}

// FP6 (sign + EB exponent + MB mantissa bits, bias BIAS, subnormal at
// exponent 0, no infinities): E2M3 = <2, 3, 1> (largest 7.5), E3M2 =
// <3, 2, 3> (largest 28).
template <int EB, int MB, int BIAS>
struct Fp6Fmt {
  static constexpr float vmax = (2.0f - 1.0f / (float)(1 << MB)) * (float)(1 << ((1 << EB) - 1 - BIAS));
  static constexpr float sub_scale = (float)(1 << (BIAS - 1 + MB));    // 1 / subnormal spacing
  static constexpr float zero_below = 0.5f / sub_scale;                  // half the smallest subnormal
};

// Tiled 6-bit storage: rows in blocks of 32 (padded with zero codes); the 32
// codes of (row, group g, 64-wide step s, half h) -- k = 128 g + 64 s + 32 h
// + j -- form a 192-bit little-endian string (code j at bits 6 j), cut into
// three 8-byte pieces u; piece u of row 32 b + r lives at byte
// ((2 s + h) * 3 + u) * 256 + 8 r of record (b, g), 3072 bytes, records in
// (b, g) order.  A matrix operand (one lane half, one step) is then three
// 8-byte reads that 32 lanes take from 256 contiguous bytes.
constexpr int kX6Record = 3072;

typedef float f32x16v __attribute__((ext_vector_type(16)));
typedef uint32_t u32x6v __attribute__((ext_vector_type(6)));

// Keeps both sources of a packed FP6 conversion live past its result w.  The
// compiler may otherwise give the conversion's six result registers to a
// source that ends there, and the instruction writes its first result dwords
// before it has read all of its first source: with the result in registers
// 4..9 of the first source, code 8 came out wrong.  Sources still live where
// the result is defined cannot share registers with it (the empty asm takes
// the result too, so it stays after the conversion).
__device__ __forceinline__ void fp6_keep_sources(u32x6v& w, const f32x16v& ev, const f32x16v& od) {
  asm volatile("" : "+v"(w) : "v"(ev), "v"(od));
}

// The three 8-byte pieces of one 32-value unit (bf16 values in t) at rec.
// r = x / s (correctly rounded) goes through the packed FP6 conversion
// instruction (unit scale; round to nearest even, saturating at the largest
// value), which packs its two 16-value operands interleaved (output j from
// operand j % 2, element j / 2): even values in the first, odd in the
// second give code j at bits 6 j.  Values that round to zero are set to +0
// first (the instruction keeps the sign of zero).
template <int EB, int MB, int BIAS>
__device__ __forceinline__ void fp6_unit(const u32x4 (&t)[4], bool zero, bool fast, float s, float y,
                                         uint8_t* rec, int un) {
  float r[32];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int e = 0; e < 8; ++e) r[8 * i + e] = bf16_bits_to_f32((e & 1) ? (t[i][e >> 1] >> 16) : (t[i][e >> 1] & 0xFFFFu));
  quotients<32>(r, zero, fast, s, y);
  f32x16v ev, od;
#pragma unroll
  for (int j = 0; j < 32; ++j) {
    const float v = __builtin_fabsf(r[j]) <= Fp6Fmt<EB, MB, BIAS>::zero_below ? 0.0f : r[j];
    if (j & 1) od[j >> 1] = v; else ev[j >> 1] = v;
  }
  u32x6v w;
  if constexpr (EB == 2)
    w = __builtin_bit_cast(u32x6v, __builtin_amdgcn_cvt_scalef32_2xpk16_fp6_f32(ev, od, 1.0f));
  else
    w = __builtin_bit_cast(u32x6v, __builtin_amdgcn_cvt_scalef32_2xpk16_bf6_f32(ev, od, 1.0f));
  fp6_keep_sources(w, ev, od);
#pragma unroll
  for (int u = 0; u < 3; ++u) {
    const u32x2 piece = {w[2 * u], w[2 * u + 1]};
    *reinterpret_cast<u32x2*>(rec + (un >> 2) * kX6Record + ((un & 3) * 3 + u) * 256) = piece;
  }
}

// Sixteen rows per workgroup of 16 waves (rows up to m_pad; padding rows
// get zero codes and no scale).  The storage interleaves 32 rows at 8-byte
// granularity, so the unit of work that writes whole cache lines is one
// 32-value unit of 16 consecutive rows (128 bytes per piece).  Pass 1: wave w
// reads row w (coalesced) for its abs-max and scale and, for rows of up to
// kRow6Lds values, parks it in LDS.  Pass 2: lane t converts unit t / 16
// (+ 64 j) of row t % 16 -- from LDS, or for wider rows again from memory
// (the rows were just read) -- and stores its pieces.
constexpr int kRow6Lds = 4096;
template <int EB, int MB, int BIAS, bool IN_LDS>
__global__ __launch_bounds__(1024) void fp6_quantize_rows_kernel(const uint16_t* __restrict__ x, int64_t m, int k,
                                                                uint8_t* __restrict__ q, float* __restrict__ sx) {
  __shared__ float srow[16], yrow[16];
  __shared__ __attribute__((aligned(16))) uint16_t buf[IN_LDS ? 16 : 1][IN_LDS ? kRow6Lds + 8 : 8];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int64_t row0 = (int64_t)blockIdx.x * 16;
  const int G = k / 128, units = k / 32;
  {
    const int64_t row = row0 + wave;
    float a = 0.0f;
    if (row < m) {
      const u32x4* src = reinterpret_cast<const u32x4*>(x + row * k);
#pragma unroll 4
      for (int c = lane; c < k / 8; c += 64) {
        const u32x4 t = src[c];
        if constexpr (IN_LDS) *reinterpret_cast<u32x4*>(&buf[wave][c * 8]) = t;
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          a = __builtin_fmaxf(a, __builtin_fabsf(bf16_bits_to_f32(t[j] & 0xFFFFu)));
          a = __builtin_fmaxf(a, __builtin_fabsf(bf16_bits_to_f32(t[j] >> 16)));
        }
      }
#pragma unroll
      for (int off = 32; off >= 1; off >>= 1) a = __builtin_fmaxf(a, __shfl_xor(a, off));
    } else if constexpr (IN_LDS) {
      for (int c = lane; c < k / 8; c += 64) *reinterpret_cast<u32x4*>(&buf[wave][c * 8]) = u32x4{0u, 0u, 0u, 0u};
    }
    if (lane == 0) {
      const float sc = a / Fp6Fmt<EB, MB, BIAS>::vmax;
      srow[wave] = sc;
      yrow[wave] = markstein_ok(sc) ? 1.0f / sc : 0.0f;
      if (row < m) sx[row] = sc;
    }
  }
  __syncthreads();
  const int r = tid & 15;
  const float s = srow[r], y = yrow[r];
  const bool zero = !(s != 0.0f), fast = markstein_ok(s);
  const int64_t row = row0 + r;
  uint8_t* rec = q + (row >> 5) * (int64_t)G * kX6Record + (row & 31) * 8;
  for (int un = tid >> 4; un < units; un += 64) {
    u32x4 t[4];
    if constexpr (IN_LDS) {
#pragma unroll
      for (int c = 0; c < 4; ++c) t[c] = *reinterpret_cast<const u32x4*>(&buf[r][un * 32 + c * 8]);
    } else {
#pragma unroll
      for (int c = 0; c < 4; ++c)
        t[c] = row < m ? *reinterpret_cast<const u32x4*>(x + row * k + un * 32 + c * 8) : u32x4{0u, 0u, 0u, 0u};
    }
    fp6_unit<EB, MB, BIAS>(t, zero, fast, s, y, rec, un);
  }
}

// FP6 weights: one lane per 32-weight chunk (the 4 lanes of a 128-group are
// adjacent: the group abs-max is a 2-step butterfly inside the quad), scale
// fl32(amax / vmax) (the smallest power of two at least that with POW2),
// r = w / s correctly rounded, codes by the packed FP6 conversion (as
// fp6_unit).  Chunk j of a row's group g is its unit (step j / 2, half
// j % 2); it goes to record (row / 32, g) of the tiled 6-bit storage with
// the weight rows in place of tokens; the scales go 32 per (row block,
// group), row 32 b + r at position r.  Chunks n_in .. n_out - 1 (padding
// rows) read no input and write zero codes and scales.
template <int EB, int MB, int BIAS, bool F32_IN, bool POW2>
__global__ __launch_bounds__(256) void fp6w_quantize_pack_kernel(const void* __restrict__ w, int64_t n_in,
                                                                int64_t n_out, int cpr, uint8_t* __restrict__ q,
                                                                float* __restrict__ scales) {
  const int64_t c = (int64_t)blockIdx.x * 256 + threadIdx.x;
  const bool valid = c < n_out;
  const bool has_src = c < n_in;
  const int64_t cc = has_src ? c : 0;
  float v[32];
  if (!has_src) {
#pragma unroll
    for (int i = 0; i < 32; ++i) v[i] = 0.0f;
  } else if constexpr (F32_IN) {
    const f32x4* src = reinterpret_cast<const f32x4*>(static_cast<const float*>(w) + cc * 32);
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const f32x4 t = src[i];
      v[4 * i] = t[0]; v[4 * i + 1] = t[1]; v[4 * i + 2] = t[2]; v[4 * i + 3] = t[3];
    }
  } else {
    const u32x4* src = reinterpret_cast<const u32x4*>(static_cast<const uint16_t*>(w) + cc * 32);
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
  float a = 0.0f;
#pragma unroll
  for (int i = 0; i < 32; ++i) a = __builtin_fmaxf(a, __builtin_fabsf(v[i]));
  a = __builtin_fmaxf(a, __shfl_xor(a, 1));
  a = __builtin_fmaxf(a, __shfl_xor(a, 2));
  float s = a / Fp6Fmt<EB, MB, BIAS>::vmax;
  if constexpr (POW2) s = pow2_at_least(s);
  const bool zero = !(s != 0.0f);
  f32x16v ev, od;
#pragma unroll
  for (int j = 0; j < 32; ++j) {
    const float r = zero ? 0.0f : v[j] / s;
    const float rv = __builtin_fabsf(r) <= Fp6Fmt<EB, MB, BIAS>::zero_below ? 0.0f : r;
    if (j & 1) od[j >> 1] = rv; else ev[j >> 1] = rv;
  }
  u32x6v wd;
  if constexpr (EB == 2)
    wd = __builtin_bit_cast(u32x6v, __builtin_amdgcn_cvt_scalef32_2xpk16_fp6_f32(ev, od, 1.0f));
  else
    wd = __builtin_bit_cast(u32x6v, __builtin_amdgcn_cvt_scalef32_2xpk16_bf6_f32(ev, od, 1.0f));
  fp6_keep_sources(wd, ev, od);
  if (valid) {
    const int64_t row = c / cpr;
    const int j = (int)(c - row * cpr);
    const int64_t G = cpr / 4, g = j >> 2;
    const int un = j & 3;
    const int64_t blk = (row >> 5) * G + g;
    const int lr = (int)(row & 31);
    uint8_t* rec = q + blk * kX6Record + lr * 8;
#pragma unroll
    for (int u = 0; u < 3; ++u) {
      const u32x2 piece = {wd[2 * u], wd[2 * u + 1]};
      *reinterpret_cast<u32x2*>(rec + (un * 3 + u) * 256) = piece;
    }
    if (un == 0) scales[blk * 32 + lr] = zero ? 0.0f : s;
  }
}

typedef int i32x8 __attribute__((ext_vector_type(8)));
typedef float f32x16e __attribute__((ext_vector_type(16)));

// X tile per 128-group: 256 rows x 128 bytes of E4M3 (32 KB); row r holds
// its 16-byte chunk c at slot c ^ xswz(r).  A ds_read_b128 serves 16 lanes
// (256 bytes, all 64 banks) per cycle: 16 consecutive rows, one chunk, must
// land on 16 distinct 16-byte bank groups, i.e. distinct slots among the
// even rows and among the odd rows (a row is half a bank line); eight
// consecutive rows get eight distinct slots as well.  The slot depends on
// r % 32 only, so every 32-row block shares the same read addresses.
__device__ __forceinline__ int xswz(int r) { return (r ^ ((r >> 3) & 1)) & 7; }
// Three stages: the DMA of group g + 2 runs while group g is multiplied.
constexpr int kW8Stage = 256 * 128;
constexpr int kW8Stages = 3;

// Workgroup = 8 waves on a 256-row tile: WM waves along M, each owning RB =
// 8 / WM row blocks of 32, times 8 / WM waves along N, each owning CB column
// blocks of 32 (tile width TN = 32 CB 8 / WM).  Per 128-group, row block and
// column block: two v_mfma_scale_f32_32x32x64_f8f6f4 (A = X as E4M3 from
// LDS, B = the packed codes straight from the weight rows).  With float32
// group scales the pair runs from zero and its partial sum is scaled by the
// column's group scale into the running accumulator (overlapping the next
// pair); with power-of-two scales (POW2) the instruction applies the scale
// itself (its B block scale, E8M0 = the scale's exponent field) and
// accumulates straight into acc.
//
// AF selects the activation operand: 0 = E4M3 rows (above), 2 = E2M3 or
// 3 = E3M2 in the tiled 6-bit storage (8 records of 3 KB per group: 24 KB
// stages, three DMAs per wave, A read as three conflict-free 8-byte pieces).
// FP6 and FP4 operands share one lane layout, so an FP6 A lane half h pairs
// element j with the FP4 B element j of the same half: both carry the
// step's k 32 h + j.
template <int FMT, bool POW2, bool TILED, int WM, int CB, int AF>
__global__ __launch_bounds__(512, 1) void w4a8_gemm_kernel(W4A8Args args) {
  constexpr int RB = 8 / WM;
  constexpr int TN = 32 * CB * (8 / WM);
  constexpr bool kA6 = AF != 0;
  static_assert(!kA6 || (FMT <= kFp4E1M2 && TILED), "6-bit activations pair with tiled FP4 weights");
  // FP6 weights (tiled 6-bit storage, a record of 3 KB per column block and
  // group) run as the B operand against E4M3 activations
  constexpr bool kW6 = FMT == kFp6wE2M3 || FMT == kFp6wE3M2;
  static_assert(!kW6 || (TILED && AF == 0), "FP6 weights: tiled storage, E4M3 activations");
  constexpr uint32_t kWRec = kW6 ? (uint32_t)kX6Record : 2048u;   // weight bytes per (block, group)
  constexpr int kWPieces = (int)kWRec / 1024;
  using BReg = std::conditional_t<kW6, u32x6v, u32x4>;
  constexpr int kStage = kA6 ? 8 * kX6Record : kW8Stage;
  constexpr int kXDma = kA6 ? 3 : 4;                     // X DMAs per wave and group
  // Several waves along M share each weight column: then the tile's weight
  // records (tiled storage) go to LDS by DMA together with X, two groups
  // ahead and once per workgroup, and every wave reads its B operands there.
  constexpr bool kBLds = TILED && WM > 1;
  constexpr int kNBlk = (8 / WM) * CB;                   // 32-column blocks per tile
  constexpr int kBStage = kBLds ? kNBlk * (int)kWRec : 0;
  constexpr int kBDma = kBLds ? (kWPieces * kNBlk + 7) / 8 : 0;  // per wave; the surplus repeats the first pieces
  // one array per stage, every stage index a compile-time constant: the
  // compiler can then tell the stage being read from the one being filled
  // and keeps the fill in flight across the barrier
  __shared__ __attribute__((aligned(1024))) uint8_t lds0[kStage];
  __shared__ __attribute__((aligned(1024))) uint8_t lds1[kStage];
  __shared__ __attribute__((aligned(1024))) uint8_t lds2[kStage];
  __shared__ __attribute__((aligned(1024))) uint8_t ldb0[kBLds ? kBStage : 16];
  __shared__ __attribute__((aligned(1024))) uint8_t ldb1[kBLds ? kBStage : 16];
  __shared__ __attribute__((aligned(1024))) uint8_t ldb2[kBLds ? kBStage : 16];
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int lane = threadIdx.x & 63;
  const int lr = lane & 31, lh = lane >> 5;
  const int wm = wave % WM, wn = wave / WM;
  int tm, tn;
  tile_coords(blockIdx.x, args.tiles_m, args.tiles_n, tm, tn);
  const int m0 = tm * 256;
  const int n0 = tn * TN;
  const int K = args.k;
  const int G = K / 128;
  const uint32_t wrow = (uint32_t)K / 2;
  const int m_valid = min(256, args.m - m0);
  const int n_valid = min(TN, args.n - n0);
  // X of this tile: 256 rows, or (6-bit) its row-block records (8 per group)
  const int rb_valid = (m_valid + 31) / 32;
  const rsrc_t rx = kA6 ? make_rsrc(args.xq + (int64_t)(m0 / 32) * G * kX6Record, (uint32_t)(rb_valid * G) * kX6Record)
                        : make_rsrc(args.xq + (int64_t)m0 * K, (uint32_t)m_valid * (uint32_t)K);
  // weights and scales of this tile's columns (tiled: its whole 32-column
  // blocks, 2048 bytes and 32 scales per block and group)
  const int nblk = (n_valid + 31) / 32;
  const rsrc_t rw = TILED ? make_rsrc(args.packed + (int64_t)(n0 / 32) * G * kWRec, (uint32_t)(nblk * G) * kWRec)
                          : make_rsrc(args.packed + (int64_t)n0 * wrow, (uint32_t)n_valid * wrow);
  const rsrc_t rs = TILED ? make_rsrc(args.wscales + (int64_t)(n0 / 32) * G * 32, (uint32_t)(nblk * G) * 128u)
                          : make_rsrc(args.wscales + (int64_t)n0 * G, (uint32_t)n_valid * G * 4);

  // X -> LDS: DMA i (0..3) of wave w fills 1 KB block 4w + i: rows
  // 8 (4w + i) + lane/8, slot lane%8 holding chunk slot ^ xswz(row).
  uint32_t xoff[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int r = 8 * (4 * wave + i) + (lane >> 3);
    const int c = (lane & 7) ^ xswz(r);
    xoff[i] = (uint32_t)r * (uint32_t)K + (uint32_t)c * 16;
  }
  // 6-bit: wave w copies record (row block w of the tile, group g), 3 KB
  const uint32_t x6off = (uint32_t)wave * (uint32_t)G * kX6Record + (uint32_t)lane * 16;
  auto issue_x = [&](int g, uint8_t* stage) __attribute__((always_inline)) {
    if constexpr (kA6) {
#pragma unroll
      for (int i = 0; i < 3; ++i)
        __builtin_amdgcn_raw_ptr_buffer_load_lds(rx, (lds_ptr_t)(stage + wave * kX6Record + i * 1024), 16,
                                                 x6off + i * 1024, (uint32_t)g * kX6Record, 0, 0);
    } else {
#pragma unroll
      for (int i = 0; i < 4; ++i)
        __builtin_amdgcn_raw_ptr_buffer_load_lds(rx, (lds_ptr_t)(stage + (4 * wave + i) * 1024), 16, xoff[i],
                                                 (uint32_t)g * 128, 0, 0);
    }
  };
  // B: the lane's column of each column block; per 64-wide step ks, lane
  // half h loads the 16 bytes (codes 32 h .. 32 h + 31 of the step) at byte
  // 32 ks + 16 h of the group's slice of the column's row, or (tiled) at
  // 1024 ks + 512 h + 16 (lane % 32) of the (block, group) record: one load
  // instruction reads 1 KB in one piece instead of 32 pieces of 32 bytes.
  //  * E2M1 runs as an FP4 B operand.  The instruction pairs B's lane half
  //    h nibbles 0-15 with A's k 16h .. 16h + 15 and nibbles 16-31 with A's
  //    k 32 + 16h .. 32 + 16h + 15 (read off it with one-hot operands), A's
  //    lane half h holding k 32h .. 32h + 31.  With B's half h carrying the
  //    step's codes 32h .. 32h + 31, A's half 0 must carry the step's X at
  //    k 0-15 and 32-47, half 1 at k 16-31 and 48-63: 16-byte chunks h, h + 2.
  //  * E3M0 and E1M2 are not matrix formats; their values are exact in E4M3,
  //    so B is FP8 (converted in registers through a byte lookup), which
  //    pairs like A: lane half h holds k 32 h .. 32 h + 31; A takes chunks
  //    2h and 2h + 1.
  //  * FP6 weights run as FP6 B operands: lane half h of step ks reads the
  //    three 8-byte pieces of its column's unit (ks, h) in the record (codes
  //    32 h .. 32 h + 31 of the step).  FP6 and FP4 operands share one lane
  //    layout (the W4A6 pairing), so A takes chunks h, h + 2 as for E2M1.
  constexpr bool kNative = FMT == kFp4E2M1 || kW6;
  uint32_t woff[CB], soff[CB];
#pragma unroll
  for (int cb = 0; cb < CB; ++cb) {
    if constexpr (TILED) {
      const uint32_t blk = (uint32_t)(wn * CB + cb);
      woff[cb] = blk * (uint32_t)G * kWRec +
                 (kW6 ? 768u * (uint32_t)lh + 8u * (uint32_t)lr : 512u * (uint32_t)lh + 16u * (uint32_t)lr);
      soff[cb] = blk * (uint32_t)G * 128u + 4u * (uint32_t)lr;
    } else {
      const uint32_t ncol = (uint32_t)(wn * 32 * CB + cb * 32 + lr);
      woff[cb] = ncol * wrow + 16u * (uint32_t)lh;
      soff[cb] = ncol * (uint32_t)G * 4;
    }
  }
  constexpr uint32_t kStepOff = TILED ? (kW6 ? 1536u : 1024u) : 32u;   // ks = 1
  constexpr uint32_t kGroupW = TILED ? kWRec : 64u, kGroupS = TILED ? 128u : 4u;
  auto load_w = [&](int g, BReg (&b)[CB][2], float (&sc)[CB]) __attribute__((always_inline)) {
    if constexpr (!kBLds) {
#pragma unroll
      for (int cb = 0; cb < CB; ++cb)
#pragma unroll
        for (int ks = 0; ks < 2; ++ks) {
          if constexpr (kW6) {
#pragma unroll
            for (int u = 0; u < 3; ++u) {
              const u32x2 t = __builtin_bit_cast(u32x2, __builtin_amdgcn_raw_buffer_load_b64(
                                                            rw, woff[cb] + kStepOff * ks + 256u * u,
                                                            (uint32_t)g * kGroupW, 0));
              b[cb][ks][2 * u] = t[0];
              b[cb][ks][2 * u + 1] = t[1];
            }
          } else {
            b[cb][ks] = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(
                                                      rw, woff[cb] + kStepOff * ks, (uint32_t)g * kGroupW, 0));
          }
        }
    }
#pragma unroll
    for (int cb = 0; cb < CB; ++cb)
      sc[cb] = __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(rs, soff[cb], (uint32_t)g * kGroupS, 0));
  };
  // the tile's weight records of group g -> LDS after the X stage: DMA d
  // (0 .. kWPieces kNBlk - 1) copies 1 KB piece d % kWPieces of block
  // d / kWPieces
  auto issue_b = [&](int g, uint8_t* stage) __attribute__((always_inline)) {
    if constexpr (kBLds) {
#pragma unroll
      for (int i = 0; i < kBDma; ++i) {
        const int d = (kBDma * wave + i) % (kWPieces * kNBlk);
        __builtin_amdgcn_raw_ptr_buffer_load_lds(
            rw, (lds_ptr_t)(stage + d * 1024), 16,
            (uint32_t)(d / kWPieces) * (uint32_t)G * kWRec + (uint32_t)(d % kWPieces) * 1024u + (uint32_t)lane * 16u,
            (uint32_t)g * kWRec, 0, 0);
      }
    }
  };
  auto read_a = [&](const uint8_t* stage, int rb, int ks) __attribute__((always_inline)) -> i32x8 {
    if constexpr (kA6) {
      const uint8_t* p = stage + (wm * RB + rb) * kX6Record + (ks * 2 + lh) * 3 * 256 + lr * 8;
      const u32x2 p0 = *reinterpret_cast<const u32x2*>(p);
      const u32x2 p1 = *reinterpret_cast<const u32x2*>(p + 256);
      const u32x2 p2 = *reinterpret_cast<const u32x2*>(p + 512);
      i32x8 a;
      a[0] = (int)p0[0]; a[1] = (int)p0[1]; a[2] = (int)p1[0]; a[3] = (int)p1[1];
      a[4] = (int)p2[0]; a[5] = (int)p2[1]; a[6] = 0; a[7] = 0;
      return a;
    }
    const int r = wm * 32 * RB + rb * 32 + lr;
    const int c0 = kNative ? 4 * ks + lh : 4 * ks + 2 * lh;
    const int c1 = kNative ? c0 + 2 : c0 + 1;
    const uint8_t* base = stage + r * 128;
    const u32x4 lo = *reinterpret_cast<const u32x4*>(base + ((c0 ^ xswz(r)) * 16));
    const u32x4 hi = *reinterpret_cast<const u32x4*>(base + ((c1 ^ xswz(r)) * 16));
    i32x8 a;
    a[0] = (int)lo[0]; a[1] = (int)lo[1]; a[2] = (int)lo[2]; a[3] = (int)lo[3];
    a[4] = (int)hi[0]; a[5] = (int)hi[1]; a[6] = (int)hi[2]; a[7] = (int)hi[3];
    return a;
  };

  f32x16e acc[RB][CB];
#pragma unroll
  for (int rb = 0; rb < RB; ++rb)
#pragma unroll
    for (int cb = 0; cb < CB; ++cb)
#pragma unroll
      for (int i = 0; i < 16; ++i) acc[rb][cb][i] = 0.0f;
  f32x16e zero16;
#pragma unroll
  for (int i = 0; i < 16; ++i) zero16[i] = 0.0f;

  BReg bc[CB][2], bn[CB][2];
  float sc[CB], sn[CB];
  // Group g: fetch group g + 1's weights into (bn, sn) and group g + 2's X
  // into the stage read in g - 1 (fill), multiply stage st with (bc, sc).
  // The last groups fetch themselves again into idle stages (never read), so
  // that the body stays one straight block.
  auto step = [&](int g, const uint8_t* st, uint8_t* fill, const uint8_t* stb, uint8_t* fillb)
                  __attribute__((always_inline)) {
    load_w(min(g + 1, G - 1), bn, sn);
    __builtin_amdgcn_sched_barrier(0);           // weights before X: the wait below counts on it
    issue_x(min(g + 2, G - 1), fill);
    issue_b(min(g + 2, G - 1), fillb);
    i32x8 bop[CB][2];
#pragma unroll
    for (int cb = 0; cb < CB; ++cb)
#pragma unroll
      for (int ks = 0; ks < 2; ++ks) {
        BReg braw;
        if constexpr (kBLds && kW6) {
          const uint8_t* p = stb + (wn * CB + cb) * (int)kWRec + ks * 1536 + lh * 768 + lr * 8;
#pragma unroll
          for (int u = 0; u < 3; ++u) {
            const u32x2 t = *reinterpret_cast<const u32x2*>(p + 256 * u);
            braw[2 * u] = t[0];
            braw[2 * u + 1] = t[1];
          }
        } else if constexpr (kBLds && kA6 && !kNative) {
          // FP6 A against FP8 B: A's lane half h element j is k = 16 h + j (j < 16) or
          // 32 + 16 h + j - 16, B's is k = 32 h + j; so B's half h takes codes
          // 16 h .. 16 h + 15 of both 32-code units (8 bytes of each half's slice)
          const uint8_t* p = stb + (wn * CB + cb) * 2048 + ks * 1024 + lr * 16 + lh * 8;
          const u32x2 u0 = *reinterpret_cast<const u32x2*>(p);
          const u32x2 u1 = *reinterpret_cast<const u32x2*>(p + 512);
          braw = u32x4{u0[0], u0[1], u1[0], u1[1]};
        } else if constexpr (kBLds) {
          braw = *reinterpret_cast<const u32x4*>(stb + (wn * CB + cb) * 2048 + ks * 1024 + lh * 512 + lr * 16);
        } else {
          braw = bc[cb][ks];
        }
        if constexpr (kW6) {
#pragma unroll
          for (int j = 0; j < 6; ++j) bop[cb][ks][j] = (int)braw[j];
          bop[cb][ks][6] = 0;
          bop[cb][ks][7] = 0;
        } else if constexpr (kNative) {
#pragma unroll
          for (int j = 0; j < 4; ++j) {
            bop[cb][ks][j] = (int)braw[j];
            bop[cb][ks][j + 4] = 0;
          }
        } else {
#pragma unroll
          for (int j = 0; j < 4; ++j) {
            const u32x2 c = fp4_codes_to_e4m3<FMT>(braw[j]);
            bop[cb][ks][2 * j] = (int)c[0];
            bop[cb][ks][2 * j + 1] = (int)c[1];
          }
        }
      }
    int sb[CB];
#pragma unroll
    for (int cb = 0; cb < CB; ++cb) sb[cb] = (int)((__builtin_bit_cast(uint32_t, sc[cb]) >> 23) & 0xFFu);
    // B as FP6 (E2M3 2, E3M2 3), FP4 (E2M1) or FP8 (E4M3)
    constexpr int kBFmt = kW6 ? (FMT == kFp6wE2M3 ? 2 : 3) : (kNative ? 4 : 0);
    // with power-of-two scales row block rb's A reads are issued one row
    // block earlier; with float32 scales (16 more registers live for the
    // rescale) at the top of the row block, behind the previous MFMAs
    constexpr bool kPrefetchA = POW2 || kBLds;
    // float32 scales: a block's partial sum is scaled into acc while the next
    // block's MFMAs run (kPipeScale), or right after its own MFMAs where the
    // tile leaves too few registers for the second partial sum (the other
    // wave on the SIMD covers the wait)
    constexpr bool kPipeScale = RB * CB <= 4 || kBLds;
    i32x8 a0 = read_a(st, 0, 0), a1 = read_a(st, 0, 1);
    f32x16e tp;
#pragma unroll
    for (int rb = 0; rb < RB; ++rb) {
      i32x8 n0a, n1a;
      if (kPrefetchA && rb + 1 < RB) {
        n0a = read_a(st, rb + 1, 0);
        n1a = read_a(st, rb + 1, 1);
      } else if (!kPrefetchA && rb > 0) {
        a0 = read_a(st, rb, 0);
        a1 = read_a(st, rb, 1);
      }
#pragma unroll
      for (int cb = 0; cb < CB; ++cb) {
        if constexpr (POW2) {
          acc[rb][cb] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a0, bop[cb][0], acc[rb][cb], AF, kBFmt,
                                                                        0, 127, 0, sb[cb]);
          acc[rb][cb] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a1, bop[cb][1], acc[rb][cb], AF, kBFmt,
                                                                        0, 127, 0, sb[cb]);
        } else {
          f32x16e t = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a0, bop[cb][0], zero16, AF, kBFmt,
                                                                      0, 127, 0, 127);
          t = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a1, bop[cb][1], t, AF, kBFmt, 0, 127, 0, 127);
          if constexpr (kPipeScale) {
            if (rb * CB + cb > 0) {
              const int p = rb * CB + cb - 1;                // the previous block, scaled now
#pragma unroll
              for (int i = 0; i < 16; ++i)
                acc[p / CB][p % CB][i] = __builtin_fmaf(tp[i], sc[p % CB], acc[p / CB][p % CB][i]);
            }
            tp = t;
          } else {
#pragma unroll
            for (int i = 0; i < 16; ++i) acc[rb][cb][i] = __builtin_fmaf(t[i], sc[cb], acc[rb][cb][i]);
          }
        }
      }
      if (kPrefetchA && rb + 1 < RB) {
        a0 = n0a;
        a1 = n1a;
      }
      __builtin_amdgcn_sched_barrier(0);
    }
    if constexpr (!POW2 && kPipeScale) {
#pragma unroll
      for (int i = 0; i < 16; ++i)
        acc[RB - 1][CB - 1][i] = __builtin_fmaf(tp[i], sc[CB - 1], acc[RB - 1][CB - 1][i]);
    }
    // everything but this wave's DMAs of group g + 2 has landed: the next
    // group's weights and (for every wave, after the barrier) its X
    constexpr int kAhead = kXDma + kBDma;
    static_assert(kAhead < 16, "vmcnt immediate");
    __builtin_amdgcn_s_waitcnt(0x0F70 | kAhead);
    // ... and every wave is done with stage st.  A plain barrier: a release
    // fence would also wait for the X DMAs just issued.
    asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
#pragma unroll
    for (int cb = 0; cb < CB; ++cb) {
      bc[cb][0] = bn[cb][0];
      bc[cb][1] = bn[cb][1];
      sc[cb] = sn[cb];
    }
  };

  issue_x(0, lds0);
  issue_b(0, ldb0);
  issue_x(min(1, G - 1), lds1);
  issue_b(min(1, G - 1), ldb1);
  load_w(0, bc, sc);
  __builtin_amdgcn_s_waitcnt(0);
  lds_barrier();
  // three groups per trip: group g reads stage g % 3
  int g = 0;
  for (; g + 2 < G; g += 3) {
    step(g, lds0, lds2, ldb0, ldb2);
    step(g + 1, lds1, lds0, ldb1, ldb0);
    step(g + 2, lds2, lds1, ldb2, ldb1);
  }
  if (g < G) step(g, lds0, lds2, ldb0, ldb2);
  if (g + 1 < G) step(g + 1, lds1, lds0, ldb1, ldb0);
  __builtin_amdgcn_s_waitcnt(0);                 // this wave's DMAs into the idle stages landed
  __syncthreads();                               // ... every wave's, and every read is done

  // Epilogue: each 32 x 32 block, scaled by its rows' token scales, leaves
  // through a 5 KB LDS scratch per wave (waves 0-3 in stage 0, 4-7 in stage 1)
  static_assert(4 * kEpiScratch <= kStage, "epilogue scratch");
  float* scratch = reinterpret_cast<float*>((wave < 4 ? lds0 : lds1) + (wave & 3) * kEpiScratch);
  const bool vec = epi_vec_ok(args.y, args.n, args.out_bf16 != 0);
#pragma unroll
  for (int rb = 0; rb < RB; ++rb) {
    const int row0 = m0 + wm * 32 * RB + rb * 32;
    float xs[16];
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const int row = row0 + 8 * (r >> 2) + 4 * lh + (r & 3);
      xs[r] = row < args.m ? args.xscales[row] : 0.0f;
    }
#pragma unroll
    for (int cb = 0; cb < CB; ++cb) {
      f32x16e v;
#pragma unroll
      for (int r = 0; r < 16; ++r) v[r] = acc[rb][cb][r] * xs[r];
      const int col0 = n0 + wn * 32 * CB + cb * 32;
      if (args.out_bf16)
        store_block32<true>(v, scratch, args.y, args.m, args.n, row0, col0, vec);
      else
        store_block32<false>(v, scratch, args.y, args.m, args.n, row0, col0, vec);
    }
  }
}

template <int FMT, bool F32_IN, bool POW2>
hipError_t launch_fp4_quant3(int64_t n, int k, bool tiled, const void* w, uint32_t* packed, float* scales,
                             hipStream_t stream) {
  const int cpr = k / 32;
  const int64_t n_in = n * cpr;
  const int64_t n_out = tiled ? (n + 31) / 32 * 32 * cpr : n_in;
  const dim3 grid((unsigned)((n_out + 255) / 256)), block(256);
  if (tiled)
    fp4_quantize_pack_kernel<FMT, F32_IN, POW2, true><<<grid, block, 0, stream>>>(w, n_in, n_out, cpr, packed, scales);
  else
    fp4_quantize_pack_kernel<FMT, F32_IN, POW2, false><<<grid, block, 0, stream>>>(w, n_in, n_out, cpr, packed, scales);
  return hipGetLastError();
}

template <int FMT>
hipError_t launch_fp4_quant(const void* w, bool f32_in, bool pow2, bool tiled, int64_t n, int k, uint32_t* packed,
                            float* scales, hipStream_t stream) {
  if (f32_in)
    return pow2 ? launch_fp4_quant3<FMT, true, true>(n, k, tiled, w, packed, scales, stream)
                : launch_fp4_quant3<FMT, true, false>(n, k, tiled, w, packed, scales, stream);
  return pow2 ? launch_fp4_quant3<FMT, false, true>(n, k, tiled, w, packed, scales, stream)
              : launch_fp4_quant3<FMT, false, false>(n, k, tiled, w, packed, scales, stream);
}

template <int FMT, bool POW2, bool TILED, int WM, int CB, int AF = 0>
hipError_t launch_w4a8_cfg(W4A8Args a, hipStream_t stream) {
  constexpr int TN = 32 * CB * (8 / WM);
  a.tiles_m = (a.m + 255) / 256;
  a.tiles_n = (a.n + TN - 1) / TN;
  w4a8_gemm_kernel<FMT, POW2, TILED, WM, CB, AF><<<dim3((unsigned)(a.tiles_m * a.tiles_n)), dim3(512), 0, stream>>>(a);
  return hipGetLastError();
}

// Tile shapes (measured at 4096 x 3072 x 3072): E2M1 on tiled storage runs
// 4 waves along M x 2 along N, 64 rows x 96 columns each (256 x 192 tiles:
// a quarter of the LDS reads, and 256 tiles at N = 3072 fill 256 CUs); row
// storage (32 scattered pieces per operand load) and the byte-lookup formats
// (whose conversion would be repeated by every wave along M) keep one wave
// per 32 columns of all 256 rows.
template <int FMT, bool POW2>
hipError_t launch_w4a8(const W4A8Args& a, bool tiled, hipStream_t stream) {
  if constexpr (FMT == kFp4E2M1) {
    if (tiled) return launch_w4a8_cfg<FMT, POW2, true, 4, 3>(a, stream);
  }
  return tiled ? launch_w4a8_cfg<FMT, POW2, true, 1, 1>(a, stream) : launch_w4a8_cfg<FMT, POW2, false, 1, 1>(a, stream);
}

template <int FMT>
hipError_t launch_w4a8(const W4A8Args& a, bool pow2, bool tiled, hipStream_t stream) {
  return pow2 ? launch_w4a8<FMT, true>(a, tiled, stream) : launch_w4a8<FMT, false>(a, tiled, stream);
}

}  // namespace

hipError_t launch_fp4_quantize_pack(const void* w, bool f32_in, int64_t n, int k, int fmt, bool pow2, bool tiled,
                                    uint32_t* packed, float* scales, hipStream_t stream) {
  switch (fmt) {
    case kFp4E2M1: return launch_fp4_quant<kFp4E2M1>(w, f32_in, pow2, tiled, n, k, packed, scales, stream);
    case kFp4E3M0: return launch_fp4_quant<kFp4E3M0>(w, f32_in, pow2, tiled, n, k, packed, scales, stream);
    case kFp4E1M2: return launch_fp4_quant<kFp4E1M2>(w, f32_in, pow2, tiled, n, k, packed, scales, stream);
  }
  return hipErrorInvalidValue;
}

hipError_t launch_fp6_quantize_rows(const uint16_t* x, int64_t m, int k, int fmt6, uint8_t* q, float* sx,
                                    hipStream_t stream) {
  if (m == 0) return hipSuccess;
  const dim3 grid((unsigned)((m + 31) / 32 * 2)), block(1024);    // 16 rows each, up to the padded count
  const bool lds = k <= kRow6Lds;
  if (fmt6 == kFp6E2M3) {
    if (lds) fp6_quantize_rows_kernel<2, 3, 1, true><<<grid, block, 0, stream>>>(x, m, k, q, sx);
    else fp6_quantize_rows_kernel<2, 3, 1, false><<<grid, block, 0, stream>>>(x, m, k, q, sx);
  } else if (fmt6 == kFp6E3M2) {
    if (lds) fp6_quantize_rows_kernel<3, 2, 3, true><<<grid, block, 0, stream>>>(x, m, k, q, sx);
    else fp6_quantize_rows_kernel<3, 2, 3, false><<<grid, block, 0, stream>>>(x, m, k, q, sx);
  } else {
    return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

namespace {
template <int FMT>
hipError_t launch_w4a6_fmt(const W4A8Args& a, int fmt6, bool pow2, hipStream_t stream) {
  if (fmt6 == kFp6E2M3)
    return pow2 ? launch_w4a8_cfg<FMT, true, true, 4, 3, 2>(a, stream)
                : launch_w4a8_cfg<FMT, false, true, 4, 3, 2>(a, stream);
  if (fmt6 == kFp6E3M2)
    return pow2 ? launch_w4a8_cfg<FMT, true, true, 4, 3, 3>(a, stream)
                : launch_w4a8_cfg<FMT, false, true, 4, 3, 3>(a, stream);
  return hipErrorInvalidValue;
}
}  // namespace

// Tiled FP4 weights of every format (E3M0 and E1M2 as FP8 B operands).
hipError_t launch_w4a6_gemm(const W4A8Args& a, int fmt, int fmt6, bool pow2, hipStream_t stream) {
  switch (fmt) {
    case kFp4E2M1: return launch_w4a6_fmt<kFp4E2M1>(a, fmt6, pow2, stream);
    case kFp4E3M0: return launch_w4a6_fmt<kFp4E3M0>(a, fmt6, pow2, stream);
    case kFp4E1M2: return launch_w4a6_fmt<kFp4E1M2>(a, fmt6, pow2, stream);
  }
  return hipErrorInvalidValue;
}

namespace {
template <int EB, int MB, int BIAS>
hipError_t launch_fp6w_quant(const void* w, bool f32_in, bool pow2, int64_t n, int k, uint8_t* packed,
                             float* scales, hipStream_t stream) {
  const int cpr = k / 32;
  const int64_t n_in = n * cpr, n_out = (n + 31) / 32 * 32 * cpr;
  const dim3 grid((unsigned)((n_out + 255) / 256)), block(256);
  if (f32_in) {
    if (pow2) fp6w_quantize_pack_kernel<EB, MB, BIAS, true, true><<<grid, block, 0, stream>>>(w, n_in, n_out, cpr, packed, scales);
    else fp6w_quantize_pack_kernel<EB, MB, BIAS, true, false><<<grid, block, 0, stream>>>(w, n_in, n_out, cpr, packed, scales);
  } else {
    if (pow2) fp6w_quantize_pack_kernel<EB, MB, BIAS, false, true><<<grid, block, 0, stream>>>(w, n_in, n_out, cpr, packed, scales);
    else fp6w_quantize_pack_kernel<EB, MB, BIAS, false, false><<<grid, block, 0, stream>>>(w, n_in, n_out, cpr, packed, scales);
  }
  return hipGetLastError();
}
}  // namespace

hipError_t launch_fp6w_quantize_pack(const void* w, bool f32_in, int64_t n, int k, int fmt6, bool pow2,
                                     uint8_t* packed, float* scales, hipStream_t stream) {
  if (n == 0) return hipSuccess;
  if (fmt6 == kFp6E2M3) return launch_fp6w_quant<2, 3, 1>(w, f32_in, pow2, n, k, packed, scales, stream);
  if (fmt6 == kFp6E3M2) return launch_fp6w_quant<3, 2, 3>(w, f32_in, pow2, n, k, packed, scales, stream);
  return hipErrorInvalidValue;
}

// FP6 weights take the tiled E2M1 tile shape (256 x 192, weights through LDS).
hipError_t launch_w6a8_gemm(const W4A8Args& a, int fmt6, bool pow2, hipStream_t stream) {
  if (fmt6 == kFp6E2M3)
    return pow2 ? launch_w4a8_cfg<kFp6wE2M3, true, true, 4, 3>(a, stream)
                : launch_w4a8_cfg<kFp6wE2M3, false, true, 4, 3>(a, stream);
  if (fmt6 == kFp6E3M2)
    return pow2 ? launch_w4a8_cfg<kFp6wE3M2, true, true, 4, 3>(a, stream)
                : launch_w4a8_cfg<kFp6wE3M2, false, true, 4, 3>(a, stream);
  return hipErrorInvalidValue;
}

hipError_t launch_fp8_quantize_rows(const uint16_t* x, int64_t m, int k, uint8_t* q, float* sx,
                                    hipStream_t stream) {
  if (m == 0) return hipSuccess;
  const int nch = (k / 8 + 255) / 256;                 // chunks per lane with one workgroup per row
  const dim3 rows((unsigned)m), block(256);
  switch (nch) {
    case 1: fp8_quantize_rows_reg_kernel<1><<<rows, block, 0, stream>>>(x, k, q, sx); break;
    case 2: fp8_quantize_rows_reg_kernel<2><<<rows, block, 0, stream>>>(x, k, q, sx); break;
    case 3: fp8_quantize_rows_reg_kernel<3><<<rows, block, 0, stream>>>(x, k, q, sx); break;
    case 4: fp8_quantize_rows_reg_kernel<4><<<rows, block, 0, stream>>>(x, k, q, sx); break;
    case 5: case 6: case 7: case 8:
      fp8_quantize_rows_reg_kernel<8><<<rows, block, 0, stream>>>(x, k, q, sx); break;
    default:
      fp8_quantize_rows_kernel<<<dim3((unsigned)((m + 3) / 4)), dim3(256), 0, stream>>>(x, m, k, q, sx);
  }
  return hipGetLastError();
}

hipError_t launch_w4a8_gemm(const W4A8Args& a, int fmt, bool pow2, bool tiled, hipStream_t stream) {
  switch (fmt) {
    case kFp4E2M1: return launch_w4a8<kFp4E2M1>(a, pow2, tiled, stream);
    case kFp4E3M0: return launch_w4a8<kFp4E3M0>(a, pow2, tiled, stream);
    case kFp4E1M2: return launch_w4a8<kFp4E1M2>(a, pow2, tiled, stream);
  }
  return hipErrorInvalidValue;
}

}  // namespace ddg
