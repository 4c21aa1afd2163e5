// C ABI of libddg (declared in include/ddg.h): argument validation on the
// host, kernel choice, launch.  No allocation, no synchronization.
#include <algorithm>
#include <atomic>
#include <cstring>
#include <mutex>
#include <random>

#include "ddg.h"
#include "ddg_launch.hpp"

namespace {

constexpr int64_t kMaxDim = 2147483647;     // M, N fit a signed 32-bit int
constexpr int64_t kMaxK = INT64_C(1) << 20; // per-tile buffer ranges stay below 4 GiB
// The low-rank pre-pass gives 16 rows of X to each workgroup of 256 lanes, so
// a launch stays below 2^32 work-items up to this many rows.
constexpr int64_t kLowrankMaxM = (INT64_C(1) << 28) - 16;
constexpr int kMaxDevices = 64;

// Per-device facts cached on first use: 0 unknown, 1 gfx950, -1 other.
std::atomic<int> g_dev_ok[kMaxDevices];
std::atomic<int> g_dev_cus[kMaxDevices];

bool aligned(const void* p, uintptr_t a) { return (reinterpret_cast<uintptr_t>(p) & (a - 1)) == 0; }

bool bits_ok(int bits) { return bits >= 3 && bits <= 7; }

bool k_ok(int64_t k) { return k > 0 && k <= kMaxDim && k % DDG_GROUP == 0; }
// rows x k weights at one lane per 32 stay within DDG_CHUNK_WEIGHTS_MAX (k
// already checked; rows may be padded)
bool chunks_ok(int64_t rows, int64_t k) { return rows <= DDG_CHUNK_WEIGHTS_MAX / k; }

// a * b without overflow past 2^62 (byte counts stay well inside int64).
bool mul_ok(int64_t a, int64_t b) { return a >= 0 && b >= 0 && (a == 0 || b <= (INT64_C(1) << 62) / a); }

// Current device: gfx950 check and compute-unit count.
int device_info(int* cus) {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) return DDG_ERR_HIP;
  if (dev < 0 || dev >= kMaxDevices) return DDG_ERR_UNSUPPORTED;
  int ok = g_dev_ok[dev].load(std::memory_order_acquire);
  if (ok == 0) {
    hipDeviceProp_t prop;
    if (hipGetDeviceProperties(&prop, dev) != hipSuccess) return DDG_ERR_HIP;
    const bool is950 = std::strncmp(prop.gcnArchName, "gfx950", 6) == 0;
    g_dev_cus[dev].store(prop.multiProcessorCount, std::memory_order_relaxed);
    ok = is950 ? 1 : -1;
    g_dev_ok[dev].store(ok, std::memory_order_release);
  }
  if (ok < 0) return DDG_ERR_UNSUPPORTED;
  *cus = g_dev_cus[dev].load(std::memory_order_relaxed);
  return DDG_OK;
}

int hip_status(hipError_t e) { return e == hipSuccess ? DDG_OK : DDG_ERR_HIP; }

template <template <int> class F, typename... A>
hipError_t by_bits(int bits, A&&... args) {
  switch (bits) {
    case 3: return F<3>::run(args...);
    case 4: return F<4>::run(args...);
    case 5: return F<5>::run(args...);
    case 6: return F<6>::run(args...);
    case 7: return F<7>::run(args...);
  }
  return hipErrorInvalidValue;
}

template <int B>
struct QuantizeF {
  template <typename... A>
  static hipError_t run(A... a) { return ddg::launch_quantize_pack<B>(a...); }
};
template <int B>
struct DequantizeF {
  template <typename... A>
  static hipError_t run(A... a) { return ddg::launch_dequantize<B>(a...); }
};
template <int B>
struct LargeF {
  template <typename... A>
  static hipError_t run(A... a) { return ddg::launch_gemm_large<B>(a...); }
};
template <int B>
struct N192F {
  template <typename... A>
  static hipError_t run(A... a) { return ddg::launch_gemm_n192<B>(a...); }
};
template <int B>
struct SmallSplitF {
  template <typename... A>
  static hipError_t run(A... a) { return ddg::launch_gemm_small_split<B>(a...); }
};
template <int B>
struct SkinnyF {
  template <typename... A>
  static hipError_t run(A... a) { return ddg::launch_gemm_skinny<B>(a...); }
};
template <int B>
struct SmallF {
  template <typename... A>
  static hipError_t run(A... a) { return ddg::launch_gemm_small<B>(a...); }
};

// Validation shared by the two GEMM entry points.
int check_gemm(const void* x, int64_t m, int64_t k, const uint8_t* packed, const float* scales,
               int bits, int64_t n, const void* y, int y_dtype) {
  if (!bits_ok(bits) || (y_dtype != DDG_BF16 && y_dtype != DDG_F32)) return DDG_ERR_ARG;
  if (m < 0 || m > kMaxDim || !k_ok(k) || k > kMaxK || n <= 0 || n > kMaxDim || n % 16)
    return DDG_ERR_SHAPE;
  if (!mul_ok(m, k) || !mul_ok(n, k) || !mul_ok(m, n)) return DDG_ERR_SHAPE;
  if (m == 0) return DDG_OK;
  if (!x || !packed || !scales || !y) return DDG_ERR_ARG;
  if (!aligned(x, 16) || !aligned(packed, 16) || !aligned(y, 16) || !aligned(scales, 4))
    return DDG_ERR_ALIGN;
  return DDG_OK;
}

// Groups per wave chunk of the M <= 16 weight-streaming kernels for K = 128 g:
// the size (5, 4 or 3) that pads the busiest wave's share of K (ceil(g / 8)
// groups) with the fewest empty groups.
int skinny_chunk(int g) {
  const int per_wave = (g + 7) / 8;
  int kc = 5, waste = 1 << 30;
  for (int c = 5; c >= 3; --c) {
    const int w = (per_wave + c - 1) / c * c - per_wave;
    if (w < waste) { waste = w; kc = c; }
  }
  return kc;
}

template <int B>
struct StreamKF {
  template <typename... A>
  static hipError_t run(A... a) { return ddg::launch_gemm_streamk<B>(a...); }
};

// Stream-K for the large-M product: one workgroup per compute unit, at most
// kSkMaxGrid (the workspace is sized for that many partial slots).
constexpr int kSkMaxGrid = 256;
constexpr size_t kSkSlotBytes = (size_t)ddg::kSkSlotFloats * sizeof(float);

size_t align256(size_t b) { return (b + 255) / 256 * 256; }

int streamk_grid(int cus) { return std::min(cus, kSkMaxGrid) / ddg::kSkXcds * ddg::kSkXcds; }

// K split across workgroups, from timings of 512- to 8192-token products of
// the DiT shapes (whole tiles against each form):
//   * split-K with `split` aligned K chunks when at most half the compute
//     units would hold a tile: split x tiles workgroups, each chunk at least
//     6 groups (so the exchange of partial sums stays small next to the work),
//     at most 8 chunks;
//   * stream-K for more tiles than workgroup slots (up to four per slot)
//     when its even spread saves at least 30% of the iterations on the
//     busiest compute unit (e.g. 320 tiles on 256 units: 241 us whole, 213
//     stream-K); with fewer tiles than slots, the exchange and the staggered
//     K positions (which defeat L2 sharing) cost more than the spread gains
//     (192 tiles of K = 3072: 90 us whole, 105 stream-K; 160 tiles of K =
//     5120: 112 us whole, 133 stream-K);
//   * else whole tiles (0).
// Returns the K chunks per tile (> 1: split-K), -1 for stream-K, 0 for tiles.
int k_split_form(int64_t tiles, int groups, int grid) {
  if (grid < ddg::kSkXcds || tiles < 1) return 0;
  if (2 * tiles <= grid) {
    const int split = (int)std::min<int64_t>({grid / tiles, groups / 6, ddg::kSkMaxSplit});
    return split >= 2 ? split : 0;
  }
  if (tiles <= grid || tiles >= 4 * (int64_t)grid) return 0;
  const double whole = (double)((tiles + grid - 1) / grid) * groups;
  const double spread = (double)tiles * groups / grid;
  return spread <= 0.7 * whole ? -1 : 0;
}

// 256 x 192 tiles (K2n) instead of 256 x 256 (whole tiles, or stream-K when
// form is -1), from interleaved timings: a round of 256 x 192 tiles over the
// compute units takes about 0.79 of a round of 256 x 256 tiles, and stream-K
// costs about 1.45 rounds per (tiles / units) (4096 x 5120 x 5120: 320 tiles,
// 214 us against 236 us for two whole rounds).  K2n is taken when its rounds
// come to at most 0.95 of the 256 x 256 plan's: 4096 x 3072 x 3072 (192
// tiles of 256 x 256, 256 of 256 x 192: 69 against 72 us), 4096 x 3072 x
// 12288 (278 against 292 us), 4096 x 5120 x 5120; not 4096 x 12288 x 3072
// (3 rounds against 4: 256 against 269 us) nor 32760 x 5120 x 5120.
bool prefer_n192(int64_t tiles256, int64_t tiles192, int form, int cus) {
  if (cus <= 0) return false;
  const double t256 = form < 0 ? 1.45 * (double)tiles256 / cus : (double)((tiles256 + cus - 1) / cus);
  const double t192 = 0.79 * (double)((tiles192 + cus - 1) / cus);
  return t192 <= 0.95 * t256;
}

// Workspace bytes of stream-K for an m x n output (0 where it is never used).
size_t streamk_bytes(int64_t m, int64_t n) {
  if (m <= 64) return 0;
  const int64_t tiles = ((m + ddg::kBM - 1) / ddg::kBM) * ((n + ddg::kBN - 1) / ddg::kBN);
  if (tiles >= 4 * (int64_t)kSkMaxGrid) return 0;
  return align256(kSkMaxGrid * kSkSlotBytes + kSkMaxGrid * sizeof(unsigned long long));
}

// The 16-token products that the skinny kernel does not take (fewer than
// 200 workgroups of 64 columns) split K across workgroups when K is long (at
// least 64 groups) and a workspace is given: 8 parts, column blocks in pairs
// (two waves per workgroup).  Interleaved timings at 16 tokens, bf16 Y:
// 5120 x 13824 (b = 5) 30.5 -> 24.5 us and 2048 x 8192 10.3 -> 9.2 us; with
// shorter K the exchange costs what the spread saves (5120 x 5120: 10.8 us
// whole, 11.1-11.8 split; 3072 x 3072 7.8 against 7.7-8.9; 1024 x 5120 7.51
// against 7.54), and 4 column blocks per workgroup or 2, 4 or 16 parts were
// no better.
constexpr int kSplitNc = 2;
int small_parts(int groups) { return groups >= 64 ? ddg::kSmallMaxParts : 1; }
bool skinny_takes(int64_t m, int64_t n) { return m <= 16 && ((n + 15) / 16) / 4 >= 200; }

// Workspace bytes of the split 16-token product (kSmallMaxParts parts of
// every column block, padded to 4 blocks; 0 where it is never used).
size_t small_split_bytes(int64_t m, int64_t n, int64_t k) {
  if (m > 16 || skinny_takes(m, n) || small_parts((int)(k / DDG_GROUP)) < 2) return 0;
  const int64_t nb4 = ((n + 15) / 16 + 3) / 4 * 4;
  return align256((size_t)nb4 * ddg::kSmallMaxParts * 1024) + align256((size_t)nb4 * ddg::kSmallMaxParts * 8);
}

// Launch epochs: unique per launch, never zero, from a random start (so a
// fresh workspace's contents are not mistaken for a published flag).
std::atomic<unsigned long long> g_epoch{0};
std::once_flag g_epoch_once;
unsigned long long next_epoch() {
  std::call_once(g_epoch_once, [] {
    std::random_device rd;
    const unsigned long long seed = ((unsigned long long)rd() << 32) ^ rd();
    g_epoch.store(seed | 1ull);
  });
  unsigned long long e = g_epoch.fetch_add(1);
  return e ? e : g_epoch.fetch_add(1);
}

// Scratch a product may use beyond its inputs and outputs (null: none).
struct Scratch {
  void* p = nullptr;
  size_t bytes = 0;
};

// Kernel choice for the product; fills a.tiles_* for the large kernel.
hipError_t launch_product(ddg::GemmArgs& a, int bits, hipStream_t stream, Scratch sk = {}, int cus = 0) {
  if (a.m <= 16) {
    // Wide outputs (at least 200 workgroups of 64 columns): the
    // weight-streaming kernel with an 8-way K split and X in registers.  Below
    // that it would either leave compute units idle or reload X (16 K bf16)
    // into too many workgroups; the LDS-ring kernel below is faster there.
    const int64_t nb = ((int64_t)a.n + 15) / 16;
    const int g = a.k / DDG_GROUP;
    if (skinny_takes(a.m, a.n)) {
      int ncb = 4;
      int kc = skinny_chunk(g);
      // shrink until the weight buffers and the scale areas fit in LDS
      auto lds = [&] { return ddg::skinny_static_lds(bits, kc, ncb) + ddg::skinny_scale_lds(kc); };
      while (lds() > ddg::kLdsLimit && (ncb > 1 || kc > 3)) {
        if (ncb > 1) ncb /= 2; else --kc;
      }
      if (lds() <= ddg::kLdsLimit) return by_bits<SkinnyF>(bits, a, kc, ncb, stream);
    }
  }
  if (a.m <= 16 && sk.p != nullptr && cus > 0) {
    const int64_t nb = ((int64_t)a.n + 15) / 16;
    const int parts = small_parts(a.k / DDG_GROUP);
    const size_t need = small_split_bytes(a.m, a.n, a.k);
    if (parts > 1 && need > 0 && sk.bytes >= need) {
      const int64_t nb4 = (nb + 3) / 4 * 4;
      ddg::SmallSplit sp{};
      sp.partials = static_cast<float*>(sk.p);
      sp.flags = reinterpret_cast<unsigned long long*>(static_cast<uint8_t*>(sk.p) +
                                                       align256((size_t)nb4 * ddg::kSmallMaxParts * 1024));
      sp.epoch = next_epoch();
      sp.parts = parts;
      return by_bits<SmallSplitF>(bits, a, kSplitNc, sp, stream);
    }
  }
  if (a.m <= 64) {
    const int rb = a.m <= 16 ? 1 : (a.m <= 32 ? 2 : 4);
    // Column waves x K-split waves per workgroup, from timings of the 16-,
    // 32- and 64-token products: four column waves where that still leaves
    // about 200+ workgroups (wide outputs; 16 tokens), two where 128+ remain
    // (with a four-way K split at 16 tokens: 16 x 5120 x 5120 10.7 us against
    // 11.8 with two), else one column wave and an 8-way (16 tokens) or 4-way
    // K split.
    const int64_t nb = ((int64_t)a.n + 15) / 16;
    int nc = 1, nk = rb == 1 ? 8 : 4;
    if (rb == 1 && nb / 4 >= 200) {
      nc = 4; nk = 2;
    } else if (nb / 2 >= 128) {
      nc = 2; nk = rb == 1 ? 4 : 2;
    }
    return by_bits<SmallF>(bits, a, rb, nc, nk, stream);
  }
  // large kernel: 256 x 256 tiles
  a.tiles_m = (a.m + ddg::kBM - 1) / ddg::kBM;
  a.tiles_n = (a.n + ddg::kBN - 1) / ddg::kBN;
  const int64_t tiles = (int64_t)a.tiles_m * a.tiles_n;
  if (tiles > kMaxDim) return hipErrorInvalidValue;
  const int grid_max = streamk_grid(cus);
  const int form = sk.p != nullptr ? k_split_form(tiles, a.k / DDG_GROUP, grid_max) : 0;
  if (form <= 0) {
    const int tn192 = (int)((a.n + ddg::kBN192 - 1) / ddg::kBN192);
    if (prefer_n192(tiles, (int64_t)a.tiles_m * tn192, form, cus)) {
      a.tiles_n = tn192;
      return by_bits<N192F>(bits, a, stream);
    }
  }
  if (form != 0 && sk.bytes >= (size_t)grid_max * kSkSlotBytes + (size_t)grid_max * sizeof(unsigned long long)) {
    ddg::StreamK k{};
    k.partials = static_cast<float*>(sk.p);
    k.flags = reinterpret_cast<unsigned long long*>(static_cast<uint8_t*>(sk.p) + (size_t)grid_max * kSkSlotBytes);
    k.epoch = next_epoch();
    k.wpx = grid_max / ddg::kSkXcds;
    k.split = form > 0 ? form : 0;
    const int grid = form > 0 ? form * (int)tiles : grid_max;
    return by_bits<StreamKF>(bits, a, k, grid, stream);
  }
  return by_bits<LargeF>(bits, a, stream);
}

// Bytes of the low-rank intermediate T (M x r bf16), rounded up to 256.
size_t lowrank_t_bytes(int64_t m, int r) { return (size_t)((m * r * 2 + 255) / 256 * 256); }

// Float32 partials of the pre-pass split over K (at most 64 rows, at least 8
// groups; chunks x M x r floats), rounded up to 256; 0 where it does not split.
size_t lowrank_part_bytes(int64_t m, int64_t k, int r) {
  if (m <= 0 || m > 64 || k / DDG_GROUP < 8 || r <= 0) return 0;
  int gpc = 1;
  const int chunks = ddg::lowrank_split_chunks((int)k, &gpc);
  return align256((size_t)chunks * (size_t)m * (size_t)r * 4);
}

// T = bf16(X L1) into t, then the product with the branch in its epilogue.
// The scratch sk (after T) holds the product's split-K area first; where room
// is left after it for the pre-pass's partials, the pre-pass splits K over
// workgroups (they are read before the product starts, in stream order).
hipError_t launch_lowrank(const void* x, int64_t m, int64_t k, const uint8_t* packed, const float* scales,
                          int bits, int64_t n, const void* lora_down, const void* lora_up, int r, void* y,
                          int y_dtype, __bf16* t, hipStream_t stream, Scratch sk = {}, int cus = 0) {
  const size_t split_area = std::max(streamk_bytes(m, n), small_split_bytes(m, n, k));
  const size_t part_bytes = lowrank_part_bytes(m, k, r);
  if (part_bytes > 0 && sk.p != nullptr && sk.bytes >= split_area + part_bytes) {
    float* part = reinterpret_cast<float*>(static_cast<uint8_t*>(sk.p) + split_area);
    if (hipError_t e = ddg::launch_lowrank_t_split(static_cast<const __bf16*>(x),
                                                   static_cast<const __bf16*>(lora_down), t, part,
                                                   (int)m, (int)k, r, stream))
      return e;
  } else if (hipError_t e = ddg::launch_lowrank_t(static_cast<const __bf16*>(x),
                                                  static_cast<const __bf16*>(lora_down), t, (int)m,
                                                  (int)k, r, stream)) {
    return e;
  }
  ddg::GemmArgs a{};
  a.x = static_cast<const __bf16*>(x);
  a.packed = packed;
  a.scales = scales;
  a.y = y;
  a.t = t;
  a.lora_up = static_cast<const __bf16*>(lora_up);
  a.m = (int)m; a.n = (int)n; a.k = (int)k; a.r = r;
  a.out_bf16 = y_dtype == DDG_BF16;
  return launch_product(a, bits, stream, sk, cus);
}

}  // namespace

extern "C" {

int ddg_version(void) { return DDG_VERSION; }

const char* ddg_status_string(int status) {
  switch (status) {
    case DDG_OK: return "ok";
    case DDG_ERR_ARG: return "invalid argument (null pointer, dtype or bit width)";
    case DDG_ERR_SHAPE: return "invalid shape";
    case DDG_ERR_ALIGN: return "misaligned pointer";
    case DDG_ERR_WORKSPACE: return "workspace too small";
    case DDG_ERR_HIP: return "HIP launch or query failed";
    case DDG_ERR_UNSUPPORTED: return "current device is not gfx950";
  }
  return "unknown status";
}

int ddg_packed_bytes(int64_t n, int64_t k, int bits, int64_t* packed_bytes, int64_t* n_scales) {
  if (!packed_bytes || !n_scales || !bits_ok(bits)) return DDG_ERR_ARG;
  if (n < 0 || !k_ok(k) || !mul_ok(n, k) || !mul_ok(n * k, bits)) return DDG_ERR_SHAPE;
  *packed_bytes = n * k / 8 * bits;
  *n_scales = n * (k / DDG_GROUP);
  return DDG_OK;
}

int ddg_quantize_pack(const void* w, int w_dtype, int64_t n, int64_t k, int bits, uint8_t* packed,
                      float* scales, hipStream_t stream) {
  if (!bits_ok(bits) || (w_dtype != DDG_BF16 && w_dtype != DDG_F32)) return DDG_ERR_ARG;
  if (n < 0 || !k_ok(k) || !mul_ok(n, k) || !mul_ok(n * k, 4) || !chunks_ok(n, k)) return DDG_ERR_SHAPE;
  if (n == 0) return DDG_OK;
  if (!w || !packed || !scales) return DDG_ERR_ARG;
  if (!aligned(w, 16) || !aligned(packed, 16) || !aligned(scales, 4)) return DDG_ERR_ALIGN;
  int cus = 0;
  if (int st = device_info(&cus)) return st;
  const int64_t n_chunks = n * k / 32;
  return hip_status(by_bits<QuantizeF>(bits, w, w_dtype == DDG_F32, n_chunks,
                                       reinterpret_cast<uint32_t*>(packed), scales, stream));
}

int ddg_dequantize(const uint8_t* packed, const float* scales, int bits, int64_t n, int64_t k,
                   void* w_out, hipStream_t stream) {
  if (!bits_ok(bits)) return DDG_ERR_ARG;
  if (n < 0 || !k_ok(k) || !mul_ok(n, k) || !mul_ok(n * k, 2) || !chunks_ok(n, k)) return DDG_ERR_SHAPE;
  if (n == 0) return DDG_OK;
  if (!packed || !scales || !w_out) return DDG_ERR_ARG;
  if (!aligned(packed, 16) || !aligned(w_out, 16) || !aligned(scales, 4)) return DDG_ERR_ALIGN;
  int cus = 0;
  if (int st = device_info(&cus)) return st;
  return hip_status(by_bits<DequantizeF>(bits, packed, scales, n * k / 32, w_out, stream));
}

int ddg_dequant_gemm(const void* x, int64_t m, int64_t k, const uint8_t* packed,
                     const float* scales, int bits, int64_t n, void* y, int y_dtype,
                     void* workspace, size_t workspace_bytes, hipStream_t stream) {
  if (int st = check_gemm(x, m, k, packed, scales, bits, n, y, y_dtype)) return st;
  if (m == 0) return DDG_OK;
  if (workspace && !aligned(workspace, 16)) return DDG_ERR_ALIGN;
  int cus = 0;
  if (int st = device_info(&cus)) return st;
  ddg::GemmArgs a{};
  a.x = static_cast<const __bf16*>(x);
  a.packed = packed;
  a.scales = scales;
  a.y = y;
  a.t = nullptr;
  a.lora_up = nullptr;
  a.m = (int)m; a.n = (int)n; a.k = (int)k; a.r = 0;
  a.out_bf16 = y_dtype == DDG_BF16;
  Scratch sk;
  if (workspace) { sk.p = workspace; sk.bytes = workspace_bytes; }
  return hip_status(launch_product(a, bits, stream, sk, cus));
}

// Column blocks of 16 per workgroup (4, 2 or 1) of a grouped launch of
// 16-token products: the choice with the least estimated time, taken as the
// larger of the costliest workgroup and the launch's total cost per compute
// unit; a workgroup costs its packed weight and scale bytes plus half its X
// bytes (16 K bf16, read from L2 by every workgroup).  Fewer columns per
// workgroup spread products with few columns or long K over more compute
// units, at the price of more X reads.  Grouped timings at 16 tokens, bf16 Y
// (4, 2, 1 column blocks): the four block linears 63.6 / 76.4 / 116.8 us, their
// 2-way N shares 47.7 / 43.1 / 63.7, their 8-way shares 45.3 / 31.0 / 24.5,
// q, k, v as three 5120 x 5120 tensors 23.0 / 28.0 / 44.5; the estimate picks
// 4, 2, 1 and 4 of them.
int grouped_ncb(const ddg_gemm_desc* descs, const int* list, int count, int cus) {
  int best = 4;
  double best_t = 0.0;
  for (int ncb : {4, 2, 1}) {
    double worst = 0.0, total = 0.0;
    for (int j = 0; j < count; ++j) {
      const ddg_gemm_desc& d = descs[list[j]];
      const double wg_bytes = 16.0 * ncb * (double)d.k * (d.bits / 8.0 + 1.0 / DDG_GROUP * 4.0)
                              + 0.5 * 32.0 * (double)d.k;
      const double wgs = (double)((d.n + 16 * ncb - 1) / (16 * ncb));
      worst = std::max(worst, wg_bytes);
      total += wgs * wg_bytes;
    }
    const double t = std::max(worst, total / std::max(cus, 1));
    if (ncb == 4 || t < best_t) {
      best = ncb;
      best_t = t;
    }
  }
  return best;
}

int ddg_dequant_gemm_grouped(const ddg_gemm_desc* descs, int count, hipStream_t stream) {
  if (count < 0 || count > DDG_MAX_GROUPED) return DDG_ERR_SHAPE;
  if (count == 0) return DDG_OK;
  if (!descs) return DDG_ERR_ARG;
  int busy = 0;
  for (int i = 0; i < count; ++i) {
    const ddg_gemm_desc& d = descs[i];
    if (int st = check_gemm(d.x, d.m, d.k, d.packed, d.scales, d.bits, d.n, d.y, d.y_dtype))
      return st;
    busy += d.m > 0;
  }
  if (busy == 0) return DDG_OK;
  int cus = 0;
  if (int st = device_info(&cus)) return st;
  auto args_of = [](const ddg_gemm_desc& d) {
    ddg::GemmArgs a{};
    a.x = static_cast<const __bf16*>(d.x);
    a.packed = d.packed;
    a.scales = d.scales;
    a.y = d.y;
    a.t = nullptr;
    a.lora_up = nullptr;
    a.m = (int)d.m; a.n = (int)d.n; a.k = (int)d.k; a.r = 0;
    a.out_bf16 = d.y_dtype == DDG_BF16;
    return a;
  };
  // Products with M <= 16 share launches, longest workgroups first (their
  // work is about K * bits per workgroup) so that the short ones fill in.
  // Products with M > 64 share launches of the large kernel's tiles, deepest
  // K first; products with 16 < M <= 32 and 32 < M <= 64 share launches of
  // the small-M kernel's body (two column waves x a two-way K split), longest
  // workgroups first.
  int small[DDG_MAX_GROUPED], large[DDG_MAX_GROUPED], mid2[DDG_MAX_GROUPED], mid4[DDG_MAX_GROUPED];
  int n_small = 0, n_large = 0, n_mid2 = 0, n_mid4 = 0;
  for (int i = 0; i < count; ++i) {
    if (descs[i].m == 0) continue;
    if (descs[i].m <= 16) small[n_small++] = i;
    else if (descs[i].m <= 32) mid2[n_mid2++] = i;
    else if (descs[i].m <= 64) mid4[n_mid4++] = i;
    else large[n_large++] = i;
  }
  auto launch_mid = [&](int* list, int n_list, int rb) -> int {
    std::stable_sort(list, list + n_list, [&](int p, int q) {
      return descs[p].k * descs[p].bits > descs[q].k * descs[q].bits;
    });
    for (int s0 = 0; s0 < n_list; s0 += ddg::kMaxGroup) {
      ddg::GroupArgs ga{};
      ga.count = std::min(ddg::kMaxGroup, n_list - s0);
      ga.wg_start[0] = 0;
      for (int j = 0; j < ga.count; ++j) {
        const ddg_gemm_desc& d = descs[list[s0 + j]];
        ga.g[j] = args_of(d);
        ga.bits[j] = d.bits;
        const int64_t wgs = (d.n + 31) / 32;
        if (ga.wg_start[j] + wgs > kMaxDim) return DDG_ERR_SHAPE;
        ga.wg_start[j + 1] = ga.wg_start[j] + (int)wgs;
      }
      if (hipError_t e = ddg::launch_gemm_grouped_small(ga, rb, stream)) return hip_status(e);
    }
    return DDG_OK;
  };
  if (int st = launch_mid(mid2, n_mid2, 2)) return st;
  if (int st = launch_mid(mid4, n_mid4, 4)) return st;
  std::stable_sort(large, large + n_large, [&](int p, int q) { return descs[p].k > descs[q].k; });
  for (int s0 = 0; s0 < n_large; s0 += ddg::kMaxGroup) {
    ddg::GroupLargeArgs ga{};
    ga.count = std::min(ddg::kMaxGroup, n_large - s0);
    ga.tile_start[0] = 0;
    for (int j = 0; j < ga.count; ++j) {
      const ddg_gemm_desc& d = descs[large[s0 + j]];
      ga.g[j] = args_of(d);
      ga.g[j].tiles_m = (int)((d.m + ddg::kBM - 1) / ddg::kBM);
      ga.g[j].tiles_n = (int)((d.n + ddg::kBN - 1) / ddg::kBN);
      ga.bits[j] = d.bits;
      const int64_t tiles = (int64_t)ga.g[j].tiles_m * ga.g[j].tiles_n;
      if (ga.tile_start[j] + tiles > kMaxDim) return DDG_ERR_SHAPE;
      ga.tile_start[j + 1] = ga.tile_start[j] + (int)tiles;
    }
    if (hipError_t e = ddg::launch_gemm_grouped_large(ga, stream)) return hip_status(e);
  }
  std::stable_sort(small, small + n_small, [&](int p, int q) {
    return descs[p].k * descs[p].bits > descs[q].k * descs[q].bits;
  });
  for (int s0 = 0; s0 < n_small; s0 += ddg::kMaxGroup) {
    ddg::GroupArgs ga{};
    ga.count = std::min(ddg::kMaxGroup, n_small - s0);
    ga.ncb = grouped_ncb(descs, small + s0, ga.count, cus);
    ga.wg_start[0] = 0;
    for (int j = 0; j < ga.count; ++j) {
      const ddg_gemm_desc& d = descs[small[s0 + j]];
      ga.g[j] = args_of(d);
      ga.bits[j] = d.bits;
      ga.kc[j] = skinny_chunk(d.k / DDG_GROUP);
      const int64_t wgs = (d.n + 16 * ga.ncb - 1) / (16 * ga.ncb);
      if (ga.wg_start[j] + wgs > kMaxDim) return DDG_ERR_SHAPE;
      ga.wg_start[j + 1] = ga.wg_start[j] + (int)wgs;
    }
    if (hipError_t e = ddg::launch_gemm_grouped(ga, stream)) return hip_status(e);
  }
  return DDG_OK;
}

int ddg_workspace_bytes(int64_t m, int64_t n, int64_t k, int r, size_t* bytes) {
  if (!bytes) return DDG_ERR_ARG;
  if (m < 0 || m > kMaxDim || n < 0 || n > kMaxDim || k < 0 || (r != 0 && (r < 8 || r > 128 || r % 8)))
    return DDG_ERR_SHAPE;
  *bytes = (r ? lowrank_t_bytes(m, r) + lowrank_part_bytes(m, k, r) : 0) +
           std::max(streamk_bytes(m, n), small_split_bytes(m, n, k));
  return DDG_OK;
}

int ddg_lowrank_down(const void* x, int64_t m, int64_t k, const void* lora_down, int r, void* t,
                     hipStream_t stream) {
  if (m < 0 || m > kLowrankMaxM || !k_ok(k) || k > kMaxK || !mul_ok(m, k)) return DDG_ERR_SHAPE;
  if (r < 8 || r > 128 || r % 8) return DDG_ERR_SHAPE;
  if (m == 0) return DDG_OK;
  if (!x || !lora_down || !t) return DDG_ERR_ARG;
  if (!aligned(x, 16) || !aligned(lora_down, 16) || !aligned(t, 16)) return DDG_ERR_ALIGN;
  return hip_status(ddg::launch_lowrank_t(static_cast<const __bf16*>(x),
                                          static_cast<const __bf16*>(lora_down),
                                          static_cast<__bf16*>(t), (int)m, (int)k, r, stream));
}

int ddg_lowrank_fused_gemm(const void* x, int64_t m, int64_t k, const uint8_t* packed,
                           const float* scales, int bits, int64_t n, const void* lora_down,
                           const void* lora_up, int r, void* y, int y_dtype, void* workspace,
                           size_t workspace_bytes, hipStream_t stream) {
  if (int st = check_gemm(x, m, k, packed, scales, bits, n, y, y_dtype)) return st;
  if (r < 8 || r > 128 || r % 8 || m > kLowrankMaxM) return DDG_ERR_SHAPE;
  if (m == 0) return DDG_OK;
  if (!lora_down || !lora_up || !workspace) return DDG_ERR_ARG;
  if (!aligned(lora_down, 16) || !aligned(lora_up, 16) || !aligned(workspace, 16))
    return DDG_ERR_ALIGN;
  const size_t t_bytes = lowrank_t_bytes(m, r);
  if (workspace_bytes < t_bytes) return DDG_ERR_WORKSPACE;
  int cus = 0;
  if (int st = device_info(&cus)) return st;
  Scratch sk;
  if (workspace_bytes > t_bytes) {
    sk.p = static_cast<uint8_t*>(workspace) + t_bytes;
    sk.bytes = workspace_bytes - t_bytes;
  }
  return hip_status(launch_lowrank(x, m, k, packed, scales, bits, n, lora_down, lora_up, r, y, y_dtype,
                                   static_cast<__bf16*>(workspace), stream, sk, cus));
}

}  // extern "C"

// ---------------------------------------------------------------------------
// The fused low-rank product without a caller workspace: T lives in a
// file-scope device array of DDG_NOALLOC_SCRATCH_BYTES bytes.  Host code never passes
// the array's name to a kernel (on the host it is only a stand-in for the
// symbol); its device address is looked up once per device, with that device
// current, and kept.
// ---------------------------------------------------------------------------
static __device__ __align__(256) uint8_t scratch[DDG_NOALLOC_SCRATCH_BYTES];

namespace {
std::atomic<void*> g_scratch[kMaxDevices];
std::mutex g_scratch_mu;

// Device address of `scratch` on the current device (looked up on the first
// call per device).  DDG_ERR_HIP when the lookup fails.
int scratch_ptr(void** out) {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) return DDG_ERR_HIP;
  if (dev < 0 || dev >= kMaxDevices) return DDG_ERR_UNSUPPORTED;
  void* p = g_scratch[dev].load(std::memory_order_acquire);
  if (p == nullptr) {
    std::lock_guard<std::mutex> lock(g_scratch_mu);
    p = g_scratch[dev].load(std::memory_order_relaxed);
    if (p == nullptr) {
      if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || p == nullptr) return DDG_ERR_HIP;
      g_scratch[dev].store(p, std::memory_order_release);
    }
  }
  *out = p;
  return DDG_OK;
}
}  // namespace

extern "C" int ddg_lowrank_fused_gemm_noalloc(const void* x, int64_t m, int64_t k, const uint8_t* packed,
                                              const float* scales, int bits, int64_t n, const void* lora_down,
                                              const void* lora_up, int r, void* y, int y_dtype,
                                              hipStream_t stream) {
  if (int st = check_gemm(x, m, k, packed, scales, bits, n, y, y_dtype)) return st;
  if (r < 8 || r > 128 || r % 8 || m > kLowrankMaxM) return DDG_ERR_SHAPE;
  if (m == 0) return DDG_OK;
  if (!lora_down || !lora_up) return DDG_ERR_ARG;
  if (!aligned(lora_down, 16) || !aligned(lora_up, 16)) return DDG_ERR_ALIGN;
  if (lowrank_t_bytes(m, r) > (size_t)DDG_NOALLOC_SCRATCH_BYTES) return DDG_ERR_WORKSPACE;
  int cus = 0;
  if (int st = device_info(&cus)) return st;
  void* t = nullptr;
  if (int st = scratch_ptr(&t)) return st;
  return hip_status(launch_lowrank(x, m, k, packed, scales, bits, n, lora_down, lora_up, r, y, y_dtype,
                                   static_cast<__bf16*>(t), stream, Scratch{}, cus));
}

extern "C" {

int ddg_rpbh_rotate(const void* x, int x_dtype, int64_t n, int64_t d, const int32_t* perm,
                    const int8_t* signs, int h, void* out, int out_dtype, hipStream_t stream) {
  if ((x_dtype != DDG_BF16 && x_dtype != DDG_F32) || (out_dtype != DDG_BF16 && out_dtype != DDG_F32))
    return DDG_ERR_ARG;
  if (n < 0 || n > kMaxDim || d <= 0 || d % 64 || d > DDG_ROTATE_MAX_D || h < 2 ||
      h > DDG_ROTATE_MAX_H || (h & (h - 1)) || d % h || !mul_ok(n, d) || !mul_ok(n * d, 4))
    return DDG_ERR_SHAPE;
  if (n == 0) return DDG_OK;
  if (!x || !perm || !signs || !out) return DDG_ERR_ARG;
  if (!aligned(x, 16) || !aligned(out, 16) || !aligned(perm, 4)) return DDG_ERR_ALIGN;
  // in place only as the very same buffer and type; otherwise no overlap
  const uintptr_t xa = reinterpret_cast<uintptr_t>(x), oa = reinterpret_cast<uintptr_t>(out);
  const uintptr_t xb = xa + (uintptr_t)(n * d * (x_dtype == DDG_F32 ? 4 : 2));
  const uintptr_t ob = oa + (uintptr_t)(n * d * (out_dtype == DDG_F32 ? 4 : 2));
  const bool same = xa == oa && x_dtype == out_dtype;
  if (!same && xa < ob && oa < xb) return DDG_ERR_ARG;
  int cus = 0;
  if (int st = device_info(&cus)) return st;
  return hip_status(ddg::launch_rpbh_rotate(x, x_dtype == DDG_F32, n, (int)d, perm, signs, h, out,
                                            out_dtype == DDG_F32, cus, stream));
}

namespace {
// the 4-bit format in the low bits, DDG_FP4_POW2 and DDG_FP4_TILED the flags
constexpr int kFp4Flags = DDG_FP4_POW2 | DDG_FP4_TILED;
bool fp4_fmt_ok(int fmt) {
  const int f = fmt & ~kFp4Flags;
  return f >= DDG_FP4_E2M1 && f <= DDG_FP4_E1M2;
}
}  // namespace

int ddg_fp4_quantize_pack(const void* w, int w_dtype, int64_t n, int64_t k, int fmt, uint8_t* packed,
                          float* scales, hipStream_t stream) {
  if (!fp4_fmt_ok(fmt) || (w_dtype != DDG_BF16 && w_dtype != DDG_F32))
    return DDG_ERR_ARG;
  if (n < 0 || n > kMaxDim || !k_ok(k) || !mul_ok(n + 31, k) || !mul_ok((n + 31) * k, 4) ||
      !chunks_ok((n + 31) / 32 * 32, k))
    return DDG_ERR_SHAPE;
  if (n == 0) return DDG_OK;
  if (!w || !packed || !scales) return DDG_ERR_ARG;
  if (!aligned(w, 16) || !aligned(packed, 16) || !aligned(scales, 4)) return DDG_ERR_ALIGN;
  int cus = 0;
  if (int st = device_info(&cus)) return st;
  return hip_status(ddg::launch_fp4_quantize_pack(w, w_dtype == DDG_F32, n, (int)k, fmt & ~kFp4Flags,
                                                  (fmt & DDG_FP4_POW2) != 0, (fmt & DDG_FP4_TILED) != 0,
                                                  reinterpret_cast<uint32_t*>(packed), scales, stream));
}

int ddg_fp8_quantize_rows(const void* x, int64_t m, int64_t k, uint8_t* xq, float* xscales,
                          hipStream_t stream) {
  if (m < 0 || m > DDG_FP8_ROWS_MAX || !k_ok(k) || !mul_ok(m, k) || !mul_ok(m * k, 2)) return DDG_ERR_SHAPE;
  if (m == 0) return DDG_OK;
  if (!x || !xq || !xscales) return DDG_ERR_ARG;
  if (!aligned(x, 16) || !aligned(xq, 8) || !aligned(xscales, 4)) return DDG_ERR_ALIGN;
  int cus = 0;
  if (int st = device_info(&cus)) return st;
  return hip_status(ddg::launch_fp8_quantize_rows(static_cast<const uint16_t*>(x), m, (int)k, xq,
                                                  xscales, stream));
}

int ddg_fp6_quantize_rows(const void* x, int64_t m, int64_t k, int fmt6, uint8_t* xq, float* xscales,
                          hipStream_t stream) {
  if (fmt6 != DDG_FP6_E2M3 && fmt6 != DDG_FP6_E3M2) return DDG_ERR_ARG;
  if (m < 0 || m > DDG_FP6_ROWS_MAX || !k_ok(k) || !mul_ok(m + 31, k) || !mul_ok((m + 31) * k, 2))
    return DDG_ERR_SHAPE;
  if (m == 0) return DDG_OK;
  if (!x || !xq || !xscales) return DDG_ERR_ARG;
  if (!aligned(x, 16) || !aligned(xq, 16) || !aligned(xscales, 4)) return DDG_ERR_ALIGN;
  int cus = 0;
  if (int st = device_info(&cus)) return st;
  return hip_status(ddg::launch_fp6_quantize_rows(static_cast<const uint16_t*>(x), m, (int)k, fmt6, xq, xscales,
                                                  stream));
}

int ddg_w4a6_gemm(const uint8_t* xq, const float* xscales, int64_t m, int64_t k, int fmt6, const uint8_t* packed,
                  const float* wscales, int fmt, int64_t n, void* y, int y_dtype, hipStream_t stream) {
  if (fmt6 != DDG_FP6_E2M3 && fmt6 != DDG_FP6_E3M2) return DDG_ERR_ARG;
  if (!fp4_fmt_ok(fmt) || (y_dtype != DDG_BF16 && y_dtype != DDG_F32)) return DDG_ERR_ARG;
  if (!(fmt & DDG_FP4_TILED)) return DDG_ERR_ARG;                                       // tiled storage only
  if (m < 0 || m > kMaxDim || !k_ok(k) || k > kMaxK || n <= 0 || n > kMaxDim || !mul_ok(m, n) ||
      !mul_ok(m * n, 4) || !mul_ok(n, k))
    return DDG_ERR_SHAPE;
  if (m == 0) return DDG_OK;
  if (!xq || !xscales || !packed || !wscales || !y) return DDG_ERR_ARG;
  if (!aligned(xq, 16) || !aligned(packed, 16) || !aligned(xscales, 4) || !aligned(wscales, 4) ||
      !aligned(y, y_dtype == DDG_F32 ? 4 : 2))
    return DDG_ERR_ALIGN;
  int cus = 0;
  if (int st = device_info(&cus)) return st;
  ddg::W4A8Args a{};
  a.xq = xq;
  a.xscales = xscales;
  a.packed = packed;
  a.wscales = wscales;
  a.y = y;
  a.m = (int)m; a.n = (int)n; a.k = (int)k;
  a.out_bf16 = y_dtype == DDG_BF16;
  return hip_status(ddg::launch_w4a6_gemm(a, fmt & ~kFp4Flags, fmt6, (fmt & DDG_FP4_POW2) != 0, stream));
}

int ddg_fp6_quantize_pack(const void* w, int w_dtype, int64_t n, int64_t k, int fmt6, uint8_t* packed,
                          float* scales, hipStream_t stream) {
  const int f = fmt6 & ~DDG_FP4_POW2;
  if ((f != DDG_FP6_E2M3 && f != DDG_FP6_E3M2) || (w_dtype != DDG_BF16 && w_dtype != DDG_F32))
    return DDG_ERR_ARG;
  if (n < 0 || n > kMaxDim || !k_ok(k) || !mul_ok(n + 31, k) || !mul_ok((n + 31) * k, 4) ||
      !chunks_ok((n + 31) / 32 * 32, k))
    return DDG_ERR_SHAPE;
  if (n == 0) return DDG_OK;
  if (!w || !packed || !scales) return DDG_ERR_ARG;
  if (!aligned(w, 16) || !aligned(packed, 16) || !aligned(scales, 4)) return DDG_ERR_ALIGN;
  int cus = 0;
  if (int st = device_info(&cus)) return st;
  return hip_status(ddg::launch_fp6w_quantize_pack(w, w_dtype == DDG_F32, n, (int)k, f,
                                                   (fmt6 & DDG_FP4_POW2) != 0, packed, scales, stream));
}

int ddg_w6a8_gemm(const uint8_t* xq, const float* xscales, int64_t m, int64_t k, const uint8_t* packed,
                  const float* wscales, int fmt6, int64_t n, void* y, int y_dtype, hipStream_t stream) {
  const int f = fmt6 & ~DDG_FP4_POW2;
  if ((f != DDG_FP6_E2M3 && f != DDG_FP6_E3M2) || (y_dtype != DDG_BF16 && y_dtype != DDG_F32))
    return DDG_ERR_ARG;
  if (m < 0 || m > kMaxDim || !k_ok(k) || k > kMaxK || n <= 0 || n > kMaxDim || !mul_ok(m, n) ||
      !mul_ok(m * n, 4) || !mul_ok(n + 31, k))
    return DDG_ERR_SHAPE;
  if (m == 0) return DDG_OK;
  if (!xq || !xscales || !packed || !wscales || !y) return DDG_ERR_ARG;
  if (!aligned(xq, 16) || !aligned(packed, 16) || !aligned(xscales, 4) || !aligned(wscales, 4) ||
      !aligned(y, y_dtype == DDG_F32 ? 4 : 2))
    return DDG_ERR_ALIGN;
  int cus = 0;
  if (int st = device_info(&cus)) return st;
  ddg::W4A8Args a{};
  a.xq = xq;
  a.xscales = xscales;
  a.packed = packed;
  a.wscales = wscales;
  a.y = y;
  a.m = (int)m; a.n = (int)n; a.k = (int)k;
  a.out_bf16 = y_dtype == DDG_BF16;
  return hip_status(ddg::launch_w6a8_gemm(a, f, (fmt6 & DDG_FP4_POW2) != 0, stream));
}

int ddg_w4a8_gemm(const uint8_t* xq, const float* xscales, int64_t m, int64_t k, const uint8_t* packed,
                  const float* wscales, int fmt, int64_t n, void* y, int y_dtype, hipStream_t stream) {
  if (!fp4_fmt_ok(fmt) || (y_dtype != DDG_BF16 && y_dtype != DDG_F32))
    return DDG_ERR_ARG;
  if (m < 0 || m > kMaxDim || !k_ok(k) || k > kMaxK || n <= 0 || n > kMaxDim || !mul_ok(m, n) ||
      !mul_ok(m * n, 4) || !mul_ok(n, k))
    return DDG_ERR_SHAPE;
  if (m == 0) return DDG_OK;
  if (!xq || !xscales || !packed || !wscales || !y) return DDG_ERR_ARG;
  if (!aligned(xq, 16) || !aligned(packed, 16) || !aligned(xscales, 4) || !aligned(wscales, 4) ||
      !aligned(y, y_dtype == DDG_F32 ? 4 : 2))
    return DDG_ERR_ALIGN;
  int cus = 0;
  if (int st = device_info(&cus)) return st;
  ddg::W4A8Args a{};
  a.xq = xq;
  a.xscales = xscales;
  a.packed = packed;
  a.wscales = wscales;
  a.y = y;
  a.m = (int)m; a.n = (int)n; a.k = (int)k;
  a.out_bf16 = y_dtype == DDG_BF16;
  return hip_status(ddg::launch_w4a8_gemm(a, fmt & ~kFp4Flags, (fmt & DDG_FP4_POW2) != 0,
                                          (fmt & DDG_FP4_TILED) != 0, stream));
}

}  // extern "C"
