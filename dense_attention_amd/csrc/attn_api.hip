// C ABI of the fused dense attention forward (declared in include/attn.h):
// argument validation, tile-variant choice, persistent-grid sizing, KV-range
// splitting and the launches on the caller's stream.  No allocation, no
// synchronisation.
#include <hip/hip_runtime.h>

#include <cmath>
#include <cstdint>
#include <cstdio>
#include <cstring>
#include <mutex>

#include "attn.h"
#include "attn_fwd_kernel.h"
#include "attn_merge_kernel.h"

// Static scratch of attn_fwd_split_noalloc: the fp32 partials of the key
// ranges live here instead of in a caller workspace.  In host code `scratch`
// only names the symbol (a host-side stand-in, not a device address); the
// device address, one per device, comes from hipGetSymbolAddress on the entry
// point's first call on that device and is the only form host code passes on.
// Every call on a device shares that device's copy, so calls that overlap on
// one device race.  Nothing in it needs to start at zero: the partial kernel
// writes every element the merge reads.
static_assert(ATTN_NOALLOC_SCRATCH_BYTES % 256 == 0, "scratch size");
static __device__ __align__(256) unsigned char scratch[ATTN_NOALLOC_SCRATCH_BYTES];

namespace {

using attn::BF16;
using attn::F16;
using attn::Params;
using attn::Tile;

constexpr float kDefaultThreshold = 8.0f;  // log2 units
constexpr float kMaxThresholdF16 = 15.0f;  // p <= 2^15 = 32768 is finite in fp16
constexpr float kLog2e = 1.4426950408889634f;

thread_local char g_last_error[256] = "";

int fail(int status, const char* detail) {
  std::snprintf(g_last_error, sizeof(g_last_error), "%s", detail ? detail : "");
  return status;
}

typedef hipError_t (*launch_fn)(const Params&, bool causal, int grid, hipStream_t stream);
typedef hipError_t (*occ_fn)(int* blocks_per_cu);

// Causal masks use a separate instantiation.
template <class T, class TL>
hipError_t launch_impl(const Params& p, bool causal, int grid, hipStream_t stream) {
  if (causal)
    hipLaunchKernelGGL((attn::attn_fwd_kernel<T, TL, true>), dim3(grid), dim3(TL::NT), 0, stream, p);
  else
    hipLaunchKernelGGL((attn::attn_fwd_kernel<T, TL, false>), dim3(grid), dim3(TL::NT), 0, stream, p);
  return hipGetLastError();
}

template <class T, class TL>
hipError_t occupancy_impl(int* blocks) {
  return hipOccupancyMaxActiveBlocksPerMultiprocessor(blocks, attn::attn_fwd_kernel<T, TL, false>,
                                                       TL::NT, 0);
}

struct Variant {
  int id;
  int dtype;
  int D;
  int block_m;
  int block_n;
  int waves;
  int stages;
  int lds_bytes;
  int key_split;
  int soft_exp;
  launch_fn launch;
  occ_fn occupancy;
};

template <class T, int DTYPE, class TL>
constexpr Variant make_variant(int id) {
  return Variant{id, DTYPE, TL::D, TL::BM, TL::BN, TL::NW, TL::STAGES, TL::LDS_BYTES,
                 TL::KSPLIT ? 1 : 0, TL::POLY, &launch_impl<T, TL>, &occupancy_impl<T, TL>};
}

#ifndef ATTN_POLY_EVERY
#define ATTN_POLY_EVERY 4
#endif

// Tile variants; ids are stable.  8 waves (256 query rows, two groups sharing
// one K/V stream), 4 waves (128 rows, one wave per SIMD), and 8 waves with a
// key split (128 rows, each group streaming half of the keys); 64- or
// 128-key tiles.
const Variant kVariants[] = {
    make_variant<BF16, ATTN_BF16, Tile<128, 64, 8, 1>>(1),
    make_variant<F16, ATTN_F16, Tile<128, 64, 8, 1>>(2),
    make_variant<BF16, ATTN_BF16, Tile<64, 64, 4, 1>>(3),
    make_variant<F16, ATTN_F16, Tile<64, 64, 4, 1>>(4),
    make_variant<BF16, ATTN_BF16, Tile<128, 64, 4, 1>>(5),
    make_variant<F16, ATTN_F16, Tile<128, 64, 4, 1>>(6),
    make_variant<BF16, ATTN_BF16, Tile<64, 64, 8, 1>>(7),
    make_variant<F16, ATTN_F16, Tile<64, 64, 8, 1>>(8),
    make_variant<BF16, ATTN_BF16, Tile<64, 64, 8, 1, true>>(9),
    make_variant<F16, ATTN_F16, Tile<64, 64, 8, 1, true>>(10),
    make_variant<BF16, ATTN_BF16, Tile<128, 64, 8, 1, true>>(11),
    make_variant<F16, ATTN_F16, Tile<128, 64, 8, 1, true>>(12),
    make_variant<BF16, ATTN_BF16, Tile<64, 128, 8, 1>>(17),
    make_variant<F16, ATTN_F16, Tile<64, 128, 8, 1>>(18),
    make_variant<BF16, ATTN_BF16, Tile<64, 128, 8, 1, true>>(19),
    make_variant<F16, ATTN_F16, Tile<64, 128, 8, 1, true>>(20),
    // Software exp2 for one score in four (selectable, never the default).
    make_variant<BF16, ATTN_BF16, Tile<64, 64, 8, 1, true, ATTN_POLY_EVERY>>(13),
    make_variant<F16, ATTN_F16, Tile<64, 64, 8, 1, true, ATTN_POLY_EVERY>>(14),
    make_variant<BF16, ATTN_BF16, Tile<128, 64, 8, 1, false, ATTN_POLY_EVERY>>(15),
    make_variant<F16, ATTN_F16, Tile<128, 64, 8, 1, false, ATTN_POLY_EVERY>>(16),
};
constexpr int kNumVariants = sizeof(kVariants) / sizeof(kVariants[0]);

const Variant* find_variant(int id) {
  for (int i = 0; i < kNumVariants; ++i)
    if (kVariants[i].id == id) return &kVariants[i];
  return nullptr;
}

// The library's choice: the 8-wave tiling with 256-row items, unless its
// items are too few to fill the device; then the key-split tiling, whose
// 128-row items take about half as long each.  Compared in rounds of one
// workgroup per compute unit, with 10% for the key split's merge.
const Variant* default_variant(int D, int dtype, int64_t BH, int Sq, int num_cus) {
  // D = 64: 128-key tiles (half the barriers and rescale tests per key; at
  // D = 128 they do not fit the registers of two waves per SIMD).
  const int shared_id = D == 128 ? (dtype == ATTN_BF16 ? 1 : 2) : (dtype == ATTN_BF16 ? 17 : 18);
  const int split_id = D == 128 ? (dtype == ATTN_BF16 ? 11 : 12) : (dtype == ATTN_BF16 ? 19 : 20);
  const Variant* a = find_variant(shared_id);
  const Variant* k = find_variant(split_id);
  if (num_cus <= 0) num_cus = 256;
  const int64_t items_a = BH * ((Sq + a->block_m - 1) / a->block_m);
  const int64_t items_k = BH * ((Sq + k->block_m - 1) / k->block_m);
  const int64_t rounds_a = (items_a + num_cus - 1) / num_cus;
  const int64_t rounds_k = (items_k + num_cus - 1) / num_cus;
  return (rounds_k * 11 < rounds_a * 20) ? k : a;
}

// Per-device facts, read once per device.
constexpr int kMaxDevices = 64;
struct DeviceInfo {
  int num_cus = 0;
  bool is_gfx950 = false;
  int occupancy[kNumVariants] = {};
};
DeviceInfo g_devices[kMaxDevices];
std::once_flag g_device_once[kMaxDevices];

int device_info(const DeviceInfo** out) {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices)
    return fail(ATTN_ERR_DEVICE, "no current HIP device");
  std::call_once(g_device_once[dev], [dev]() {
    DeviceInfo& di = g_devices[dev];
    hipDeviceProp_t prop;
    if (hipGetDeviceProperties(&prop, dev) != hipSuccess) return;
    di.num_cus = prop.multiProcessorCount;
    di.is_gfx950 = std::strncmp(prop.gcnArchName, "gfx950", 6) == 0;
    for (int i = 0; i < kNumVariants; ++i) {
      int b = 0;
      if (kVariants[i].occupancy(&b) != hipSuccess || b < 1) b = 1;
      di.occupancy[i] = b;
    }
  });
  const DeviceInfo& di = g_devices[dev];
  if (!di.is_gfx950 || di.num_cus <= 0) return fail(ATTN_ERR_DEVICE, "current device is not gfx950");
  *out = &di;
  return ATTN_OK;
}

struct Plan {
  const Variant* var = nullptr;
  int var_index = 0;
  int n_qtiles = 0;
  int n_splits = 1;
  int split_len = 0;
  int n_items = 0;
  int grid = 0;
  int per_cu = 0;
  int num_cus = 0;
  float thr = kDefaultThreshold;
  int causal = 0;        // 0 none, else the mask is on with diagonal offset coff
  int coff = 0;
  bool empty = false;
};

constexpr int kMaxSplits = 64;
constexpr int kMinSplitKeys = 1024;

// Validation shared by every forward entry point (data pointers excluded).
// kv_splits: 1 = one range per item, 0 = choose to fill the device (needs the
// device), n > 1 = at most n ranges.
int plan_launch(int B, int H, int Sq, int Skv, int D, int dtype, float scale,
                const attn_fwd_options_t* opts, int kv_splits, bool need_device, Plan* plan) {
  if (dtype != ATTN_F16 && dtype != ATTN_BF16) return fail(ATTN_ERR_DTYPE, "dtype must be ATTN_F16 or ATTN_BF16");
  if (B < 0 || H < 0 || Sq < 0 || Skv < 0) return fail(ATTN_ERR_SHAPE, "B, H and S must be >= 0");
  if (D != 64 && D != 128) return fail(ATTN_ERR_SHAPE, "D must be 64 or 128");
  if (!std::isfinite(scale)) return fail(ATTN_ERR_SCALE, "scale must be finite");
  if (kv_splits < 0 || kv_splits > kMaxSplits) return fail(ATTN_ERR_ARG, "kv_splits must be in [0, 64]");
  if (opts) {
    for (int r : opts->reserved)
      if (r != 0) return fail(ATTN_ERR_ARG, "reserved option fields must be zero");
    if (opts->grid < 0) return fail(ATTN_ERR_ARG, "grid must be >= 0");
    if (!(opts->rescale_threshold <= 64.0f) && !(opts->rescale_threshold < 0.0f))
      return fail(ATTN_ERR_ARG, "rescale_threshold must be <= 64");
    // A kept maximum lets p reach 2^threshold, and P is rounded to the input
    // type for P·V: fp16's largest finite value is 65504 < 2^16, so an fp16 P
    // stays finite only up to threshold 15 (bf16 has fp32's exponent range).
    if (dtype == ATTN_F16 && opts->rescale_threshold > kMaxThresholdF16)
      return fail(ATTN_ERR_ARG, "rescale_threshold must be <= 15 for fp16 (P would overflow fp16)");
    if (opts->causal < 0 || opts->causal > 2) return fail(ATTN_ERR_ARG, "causal must be 0, 1 or 2");
  }
  // Rows are indexed with 32-bit integers inside a head and work items with
  // 32-bit integers overall.
  if ((int64_t)B * H * (int64_t)Sq >= (int64_t)1 << 31 || Skv >= (1 << 30))
    return fail(ATTN_ERR_SHAPE, "B*H*Sq must be < 2^31 and Skv < 2^30");

  const DeviceInfo* di = nullptr;
  if (need_device || kv_splits == 0) {
    int st = device_info(&di);
    if (st != ATTN_OK) return st;
    plan->num_cus = di->num_cus;
  }
  const Variant* var = nullptr;
  if (opts && opts->variant != 0) {
    var = find_variant(opts->variant);
    if (!var) return fail(ATTN_ERR_ARG, "unknown variant id");
    if (var->D != D || var->dtype != dtype) return fail(ATTN_ERR_ARG, "variant does not support this D/dtype");
  } else {
    var = default_variant(D, dtype, (int64_t)B * H, Sq, plan->num_cus);
  }
  plan->var = var;
  plan->var_index = (int)(var - kVariants);
  if (di) plan->per_cu = di->occupancy[plan->var_index];
  plan->thr = (opts && opts->rescale_threshold >= 0.0f) ? opts->rescale_threshold : kDefaultThreshold;
  plan->causal = opts ? opts->causal : 0;
  plan->coff = plan->causal == 2 ? opts->causal_offset : Skv - Sq;
  plan->n_qtiles = (Sq + var->block_m - 1) / var->block_m;
  plan->empty = ((int64_t)B * H * plan->n_qtiles == 0);
  if (!plan->empty && Skv == 0) return fail(ATTN_ERR_SHAPE, "queries need at least one key (Skv >= 1)");
  const int base_items = B * H * plan->n_qtiles;
  // KV ranges: whole tiles.  The library's own count (kv_splits == 0): a
  // split adds an fp32 partial round trip and a merge launch, and the more
  // compute units are busy the lower the clock each of them runs at, so it
  // pays only where the items leave most of the device idle and every range
  // stays long.  With at most a quarter of the workgroup slots taken, ranges
  // of at least kMinSplitKeys keys; with at most half, at least 4x that; no
  // more items than slots.  (Measured over B·H = 1..16, S = 1K..16K, D = 64
  // and 128: within 4% of the best fixed count, or no split, in every case.)
  int want = kv_splits;
  if (want == 0) {
    const int slots = plan->num_cus * plan->per_cu;
    want = 1;
    if (base_items > 0 && 2 * base_items <= slots) {
      const int min_keys = 4 * base_items <= slots ? kMinSplitKeys : 4 * kMinSplitKeys;
      want = slots / base_items;
      if (want > Skv / min_keys) want = Skv / min_keys;
      if (want > kMaxSplits) want = kMaxSplits;
    }
  }
  if (want < 1) want = 1;
  const int bn = var->block_n;
  int len = (Skv + want - 1) / want;
  len = ((len + bn - 1) / bn) * bn;
  if (len < bn) len = bn;
  plan->split_len = want == 1 ? (Skv > 0 ? Skv : 1) : len;
  plan->n_splits = want == 1 ? 1 : (Skv + len - 1) / len;
  if ((int64_t)base_items * plan->n_splits >= (int64_t)1 << 31) return fail(ATTN_ERR_SHAPE, "too many work items");
  plan->n_items = base_items * plan->n_splits;
  if (!need_device) return ATTN_OK;

  // Causal items differ widely in length: one workgroup per item, longest
  // first, and the hardware hands them to compute units as these free up.
  int grid = plan->causal ? plan->n_items : di->num_cus * plan->per_cu;
  if (opts && opts->grid > 0) grid = opts->grid;
  if (grid > plan->n_items) grid = plan->n_items;
  plan->grid = grid;
  return ATTN_OK;
}

bool misaligned(const void* p, uintptr_t a) { return (reinterpret_cast<uintptr_t>(p) & (a - 1)) != 0; }

attn_layout_t contiguous(int H, int S, int D) {
  return attn_layout_t{(int64_t)H * S * D, (int64_t)S * D, (int64_t)D};
}

int check_layout(const attn_layout_t& l, const char* what) {
  if (l.batch_stride < 0 || l.head_stride < 0 || l.seq_stride < 0 ||
      (l.batch_stride % 8) != 0 || (l.head_stride % 8) != 0 || (l.seq_stride % 8) != 0) {
    char buf[128];
    std::snprintf(buf, sizeof(buf), "%s strides must be >= 0 and multiples of 8 elements", what);
    return fail(ATTN_ERR_SHAPE, buf);
  }
  if (l.seq_stride >= (1 << 24)) {
    char buf[128];
    std::snprintf(buf, sizeof(buf), "%s seq_stride must be < 2^24", what);
    return fail(ATTN_ERR_SHAPE, buf);
  }
  return ATTN_OK;
}

// One forward launch: inputs with their layouts, the output (dtype or fp32
// partials) and the KV-range split.
struct Forward {
  const void* q = nullptr;
  const void* k = nullptr;
  const void* v = nullptr;
  void* o = nullptr;
  float* lse = nullptr;
  attn_layout_t ql{}, kl{}, vl{}, ol{};
  int B = 0, H = 0, Sq = 0, Skv = 0, D = 0;
  float scale = 0.f;
  int dtype = 0;
  bool o_f32 = false;
  long long o_split = 0, lse_split = 0;
};

int check_pointers(const Forward& f) {
  if (!f.q || !f.k || !f.v || !f.o) return fail(ATTN_ERR_NULL, "q, k, v and o must be non-null");
  if (misaligned(f.q, 16) || misaligned(f.k, 16) || misaligned(f.v, 16) || misaligned(f.o, 16))
    return fail(ATTN_ERR_ALIGN, "q, k, v and o must be 16-byte aligned");
  if (f.lse && misaligned(f.lse, 4)) return fail(ATTN_ERR_ALIGN, "lse must be 4-byte aligned");
  int st;
  if ((st = check_layout(f.ql, "q")) != ATTN_OK) return st;
  if ((st = check_layout(f.kl, "k")) != ATTN_OK) return st;
  if ((st = check_layout(f.vl, "v")) != ATTN_OK) return st;
  if ((st = check_layout(f.ol, "o")) != ATTN_OK) return st;
  if (f.ol.seq_stride < f.D) return fail(ATTN_ERR_SHAPE, "o seq_stride must be >= D");
  return ATTN_OK;
}

int launch_forward(const Forward& f, const Plan& plan, hipStream_t stream) {
  Params p;
  p.q = static_cast<const uint16_t*>(f.q);
  p.k = static_cast<const uint16_t*>(f.k);
  p.v = static_cast<const uint16_t*>(f.v);
  p.o = f.o;
  p.lse = f.lse;
  p.q_sb = f.ql.batch_stride; p.q_sh = f.ql.head_stride; p.q_ss = (int)f.ql.seq_stride;
  p.k_sb = f.kl.batch_stride; p.k_sh = f.kl.head_stride; p.k_ss = (int)f.kl.seq_stride;
  p.v_sb = f.vl.batch_stride; p.v_sh = f.vl.head_stride; p.v_ss = (int)f.vl.seq_stride;
  p.o_sb = f.ol.batch_stride; p.o_sh = f.ol.head_stride; p.o_ss = (int)f.ol.seq_stride;
  p.o_split = f.o_split;
  p.lse_split = f.lse_split;
  p.H = f.H;
  p.BH = f.B * f.H;
  p.Sq = f.Sq;
  p.Skv = f.Skv;
  p.n_qtiles = plan.n_qtiles;
  p.n_splits = plan.n_splits;
  p.split_len = plan.split_len;
  p.n_items = plan.n_items;
  p.xcd_remap = (!plan.causal && plan.grid % 8 == 0 && plan.grid >= 8) ? 1 : 0;
  p.o_f32 = f.o_f32 ? 1 : 0;
  p.coff = plan.coff;
  p.c = f.scale * kLog2e;
  p.thr = plan.thr;
  hipError_t e = plan.var->launch(p, plan.causal != 0, plan.grid, stream);
  if (e != hipSuccess) return fail(ATTN_ERR_LAUNCH, hipGetErrorString(e));
  return ATTN_OK;
}

template <class T, int D>
hipError_t merge_launch(const attn::MergeParams& m, hipStream_t stream) {
  constexpr int RPB = 256 / (D / 8);
  const long long blocks = (m.rows + RPB - 1) / RPB;
  hipLaunchKernelGGL((attn::attn_merge_kernel<T, D>), dim3((unsigned)blocks), dim3(256), 0, stream, m);
  return hipGetLastError();
}

int launch_merge(const float* o_parts, const float* lse_parts, int n_parts, void* o,
                 const attn_layout_t& ol, float* lse, int B, int H, int S, int D, int dtype,
                 hipStream_t stream) {
  attn::MergeParams m;
  m.o_parts = o_parts;
  m.lse_parts = lse_parts;
  m.o = o;
  m.lse = lse;
  m.o_sb = ol.batch_stride;
  m.o_sh = ol.head_stride;
  m.o_ss = (int)ol.seq_stride;
  m.n_parts = n_parts;
  m.H = H;
  m.S = S;
  m.rows = (long long)B * H * S;
  m.part_stride = m.rows * D;
  m.f32_out = dtype == ATTN_F32 ? 1 : 0;
  if (m.rows / (256 / (D / 8)) >= (1LL << 31)) return fail(ATTN_ERR_SHAPE, "too many rows to merge");
  hipError_t e;
  if (dtype == ATTN_F16)
    e = D == 64 ? merge_launch<F16, 64>(m, stream) : merge_launch<F16, 128>(m, stream);
  else
    e = D == 64 ? merge_launch<BF16, 64>(m, stream) : merge_launch<BF16, 128>(m, stream);
  if (e != hipSuccess) return fail(ATTN_ERR_LAUNCH, hipGetErrorString(e));
  return ATTN_OK;
}

// Workspace of attn_fwd_split: fp32 partial O then fp32 partial LSE, each
// 256-byte aligned.
size_t split_o_bytes(int B, int H, int S, int D, int n) {
  size_t b = (size_t)n * B * H * S * D * sizeof(float);
  return (b + 255) & ~(size_t)255;
}
size_t split_ws_bytes(int B, int H, int S, int D, int n) {
  size_t l = (size_t)n * B * H * S * sizeof(float);
  return split_o_bytes(B, H, S, D, n) + ((l + 255) & ~(size_t)255);
}

int forward(const Forward& f, const attn_fwd_options_t* opts, hipStream_t stream) {
  Plan plan;
  int st = plan_launch(f.B, f.H, f.Sq, f.Skv, f.D, f.dtype, f.scale, opts, 1, /*need_device=*/false, &plan);
  if (st != ATTN_OK) return st;
  if (plan.empty) return ATTN_OK;
  if ((st = check_pointers(f)) != ATTN_OK) return st;
  st = plan_launch(f.B, f.H, f.Sq, f.Skv, f.D, f.dtype, f.scale, opts, 1, /*need_device=*/true, &plan);
  if (st != ATTN_OK) return st;
  return launch_forward(f, plan, stream);
}

struct ScratchSlot {
  void* ptr = nullptr;
  hipError_t err = hipErrorNotInitialized;
};
ScratchSlot g_scratch[kMaxDevices];
std::once_flag g_scratch_once[kMaxDevices];

// Device address of this device's scratch (the current device must be the one
// the call runs on).
int scratch_address(void** out) {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices)
    return fail(ATTN_ERR_DEVICE, "no current HIP device");
  std::call_once(g_scratch_once[dev], [dev]() {
    ScratchSlot& sl = g_scratch[dev];
    void* ptr = nullptr;
    sl.err = hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch));
    sl.ptr = sl.err == hipSuccess ? ptr : nullptr;
  });
  const ScratchSlot& sl = g_scratch[dev];
  if (sl.err != hipSuccess || sl.ptr == nullptr) {
    char buf[200];
    std::snprintf(buf, sizeof(buf), "hipGetSymbolAddress(scratch) failed: %s", hipGetErrorString(sl.err));
    return fail(ATTN_ERR_LAUNCH, buf);
  }
  *out = sl.ptr;
  return ATTN_OK;
}

int scratch_too_small(size_t need) {
  char buf[200];
  std::snprintf(buf, sizeof(buf),
                "the key-range partials need %zu bytes; the static scratch holds %zu "
                "(use fewer kv_splits, or attn_fwd_split with a workspace)",
                need, (size_t)ATTN_NOALLOC_SCRATCH_BYTES);
  return fail(ATTN_ERR_SCRATCH, buf);
}

// attn_fwd_split and attn_fwd_split_noalloc: the partials of the key ranges
// go to the caller's workspace, or to the static scratch.
int split_forward(const void* q, const void* k, const void* v, void* o, float* lse, int B, int H,
                  int S, int D, float scale, int dtype, hipStream_t hs, int kv_splits,
                  void* workspace, size_t workspace_bytes, bool static_scratch,
                  const attn_fwd_options_t* opts) {
  Plan plan;
  int st = plan_launch(B, H, S, S, D, dtype, scale, opts, kv_splits == 0 ? 1 : kv_splits,
                       /*need_device=*/false, &plan);
  if (st != ATTN_OK) return st;
  if (plan.empty) return ATTN_OK;
  // An explicit range count fixes the scratch size before any device query.
  if (static_scratch && kv_splits > 0 && plan.n_splits > 1 &&
      split_ws_bytes(B, H, S, D, plan.n_splits) > (size_t)ATTN_NOALLOC_SCRATCH_BYTES)
    return scratch_too_small(split_ws_bytes(B, H, S, D, plan.n_splits));
  Forward f;
  f.q = q; f.k = k; f.v = v; f.o = o; f.lse = lse;
  f.B = B; f.H = H; f.Sq = S; f.Skv = S; f.D = D; f.scale = scale; f.dtype = dtype;
  f.ql = f.kl = f.vl = f.ol = contiguous(H, S, D);
  if ((st = check_pointers(f)) != ATTN_OK) return st;
  st = plan_launch(B, H, S, S, D, dtype, scale, opts, kv_splits, /*need_device=*/true, &plan);
  if (st != ATTN_OK) return st;
  if (plan.n_splits == 1) return launch_forward(f, plan, hs);
  const size_t need = split_ws_bytes(B, H, S, D, plan.n_splits);
  if (static_scratch) {
    if (need > (size_t)ATTN_NOALLOC_SCRATCH_BYTES) return scratch_too_small(need);
    if ((st = scratch_address(&workspace)) != ATTN_OK) return st;
    workspace_bytes = ATTN_NOALLOC_SCRATCH_BYTES;
  } else {
    if (!workspace) return fail(ATTN_ERR_NULL, "workspace must be non-null");
    if (misaligned(workspace, 256)) return fail(ATTN_ERR_ALIGN, "workspace must be 256-byte aligned");
    if (workspace_bytes < need)
      return fail(ATTN_ERR_ARG, "workspace is smaller than attn_fwd_split_workspace_size()");
  }
  float* o_parts = static_cast<float*>(workspace);
  float* lse_parts = reinterpret_cast<float*>(static_cast<char*>(workspace) + split_o_bytes(B, H, S, D, plan.n_splits));
  Forward part = f;
  part.o = o_parts;
  part.lse = lse_parts;
  part.ol = contiguous(H, S, D);
  part.o_f32 = true;
  part.o_split = (long long)B * H * S * D;
  part.lse_split = (long long)B * H * S;
  if ((st = launch_forward(part, plan, hs)) != ATTN_OK) return st;
  return launch_merge(o_parts, lse_parts, plan.n_splits, o, f.ol, lse, B, H, S, D, dtype, hs);
}

}  // namespace

extern "C" {

int attn_fwd_ex(const void* q, const void* k, const void* v, void* o, float* lse, int B, int H,
                int S, int D, float scale, int dtype, void* stream,
                const attn_fwd_options_t* opts) {
  g_last_error[0] = '\0';
  Forward f;
  f.q = q; f.k = k; f.v = v; f.o = o; f.lse = lse;
  f.B = B; f.H = H; f.Sq = S; f.Skv = S; f.D = D; f.scale = scale; f.dtype = dtype;
  f.ql = f.kl = f.vl = f.ol = contiguous(H, S, D);
  return forward(f, opts, static_cast<hipStream_t>(stream));
}

int attn_fwd(const void* q, const void* k, const void* v, void* o, float* lse, int B, int H,
             int S, int D, float scale, int dtype, void* stream) {
  return attn_fwd_ex(q, k, v, o, lse, B, H, S, D, scale, dtype, stream, nullptr);
}

int attn_fwd_strided(const void* q, const attn_layout_t* q_layout, const void* k,
                     const attn_layout_t* k_layout, const void* v, const attn_layout_t* v_layout,
                     void* o, const attn_layout_t* o_layout, float* lse, int B, int H, int Sq,
                     int Skv, int D, float scale, int dtype, void* stream,
                     const attn_fwd_options_t* opts) {
  g_last_error[0] = '\0';
  Forward f;
  f.q = q; f.k = k; f.v = v; f.o = o; f.lse = lse;
  f.B = B; f.H = H; f.Sq = Sq; f.Skv = Skv; f.D = D; f.scale = scale; f.dtype = dtype;
  f.ql = q_layout ? *q_layout : contiguous(H, Sq, D);
  f.kl = k_layout ? *k_layout : contiguous(H, Skv, D);
  f.vl = v_layout ? *v_layout : contiguous(H, Skv, D);
  f.ol = o_layout ? *o_layout : contiguous(H, Sq, D);
  return forward(f, opts, static_cast<hipStream_t>(stream));
}

int attn_fwd_partial(const void* q, const attn_layout_t* q_layout, const void* k,
                     const attn_layout_t* k_layout, const void* v, const attn_layout_t* v_layout,
                     float* o_part, float* lse_part, int B, int H, int Sq, int Skv, int D,
                     float scale, int dtype, void* stream, const attn_fwd_options_t* opts) {
  g_last_error[0] = '\0';
  Forward f;
  f.q = q; f.k = k; f.v = v; f.o = o_part; f.lse = lse_part;
  f.B = B; f.H = H; f.Sq = Sq; f.Skv = Skv; f.D = D; f.scale = scale; f.dtype = dtype;
  f.ql = q_layout ? *q_layout : contiguous(H, Sq, D);
  f.kl = k_layout ? *k_layout : contiguous(H, Skv, D);
  f.vl = v_layout ? *v_layout : contiguous(H, Skv, D);
  f.ol = contiguous(H, Sq, D);
  f.o_f32 = true;
  Plan plan;
  int st = plan_launch(B, H, Sq, Skv, D, dtype, scale, opts, 1, /*need_device=*/false, &plan);
  if (st != ATTN_OK) return st;
  if (plan.empty) return ATTN_OK;
  if (!lse_part) return fail(ATTN_ERR_NULL, "lse_part must be non-null");
  return forward(f, opts, static_cast<hipStream_t>(stream));
}

int attn_merge(const float* o_parts, const float* lse_parts, int n_parts, void* o,
               const attn_layout_t* o_layout, float* lse, int B, int H, int S, int D, int dtype,
               void* stream) {
  g_last_error[0] = '\0';
  if (dtype != ATTN_F16 && dtype != ATTN_BF16 && dtype != ATTN_F32)
    return fail(ATTN_ERR_DTYPE, "dtype must be ATTN_F16, ATTN_BF16 or ATTN_F32");
  if (B < 0 || H < 0 || S < 0) return fail(ATTN_ERR_SHAPE, "B, H and S must be >= 0");
  if (D != 64 && D != 128) return fail(ATTN_ERR_SHAPE, "D must be 64 or 128");
  if (n_parts < 1) return fail(ATTN_ERR_ARG, "n_parts must be >= 1");
  if ((int64_t)B * H * S >= (int64_t)1 << 31) return fail(ATTN_ERR_SHAPE, "B*H*S must be < 2^31");
  if ((int64_t)B * H * S == 0) return ATTN_OK;
  if (!o_parts || !lse_parts || !o) return fail(ATTN_ERR_NULL, "o_parts, lse_parts and o must be non-null");
  if (misaligned(o_parts, 16) || misaligned(o, 16) || misaligned(lse_parts, 4) || (lse && misaligned(lse, 4)))
    return fail(ATTN_ERR_ALIGN, "o_parts and o must be 16-byte aligned, lse arrays 4-byte aligned");
  const attn_layout_t ol = o_layout ? *o_layout : contiguous(H, S, D);
  int st = check_layout(ol, "o");
  if (st != ATTN_OK) return st;
  if (ol.seq_stride < D) return fail(ATTN_ERR_SHAPE, "o seq_stride must be >= D");
  const DeviceInfo* di = nullptr;
  if ((st = device_info(&di)) != ATTN_OK) return st;
  return launch_merge(o_parts, lse_parts, n_parts, o, ol, lse, B, H, S, D, dtype,
                      static_cast<hipStream_t>(stream));
}

size_t attn_fwd_split_workspace_size(int B, int H, int S, int D, int kv_splits) {
  if (B < 0 || H < 0 || S < 0 || (D != 64 && D != 128) || kv_splits < 0 || kv_splits > kMaxSplits) return 0;
  // With kv_splits == 0 the library may choose up to kMaxSplits ranges, but
  // never more than S / kMinSplitKeys (and at least one).
  int n = kv_splits;
  if (n == 0) {
    n = S / kMinSplitKeys;
    if (n > kMaxSplits) n = kMaxSplits;
  }
  if (n < 1) n = 1;
  return split_ws_bytes(B, H, S, D, n);
}

int attn_fwd_split(const void* q, const void* k, const void* v, void* o, float* lse, int B, int H,
                   int S, int D, float scale, int dtype, void* stream, int kv_splits,
                   void* workspace, size_t workspace_bytes, const attn_fwd_options_t* opts) {
  g_last_error[0] = '\0';
  return split_forward(q, k, v, o, lse, B, H, S, D, scale, dtype, static_cast<hipStream_t>(stream),
                       kv_splits, workspace, workspace_bytes, /*static_scratch=*/false, opts);
}

int attn_fwd_split_noalloc(const void* q, const void* k, const void* v, void* o, float* lse, int B,
                           int H, int S, int D, float scale, int dtype, void* stream, int kv_splits,
                           const attn_fwd_options_t* opts) {
  g_last_error[0] = '\0';
  return split_forward(q, k, v, o, lse, B, H, S, D, scale, dtype, static_cast<hipStream_t>(stream),
                       kv_splits, nullptr, 0, /*static_scratch=*/true, opts);
}

int attn_get_config(int B, int H, int S, int D, int dtype, const attn_fwd_options_t* opts,
                    attn_config_t* out) {
  g_last_error[0] = '\0';
  if (!out) return fail(ATTN_ERR_NULL, "out must be non-null");
  Plan plan;
  int st = plan_launch(B, H, S, S, D, dtype, 1.0f, opts, 1, /*need_device=*/true, &plan);
  if (st != ATTN_OK) return st;
  out->variant = plan.var->id;
  out->block_m = plan.var->block_m;
  out->block_n = plan.var->block_n;
  out->waves = plan.var->waves;
  out->stages = plan.var->stages;
  out->lds_bytes = plan.var->lds_bytes;
  out->work_items = plan.n_items;
  out->grid = plan.grid;
  out->workgroups_per_cu = plan.per_cu;
  out->num_cus = plan.num_cus;
  return ATTN_OK;
}

int attn_variant_count(void) { return kNumVariants; }

int attn_variant_info(int index, int* id, int* head_dim, int* dtype, int* block_m, int* block_n,
                      int* waves, int* stages, int* key_split, int* soft_exp) {
  if (index < 0 || index >= kNumVariants) return fail(ATTN_ERR_ARG, "variant index out of range");
  const Variant& v = kVariants[index];
  if (id) *id = v.id;
  if (head_dim) *head_dim = v.D;
  if (dtype) *dtype = v.dtype;
  if (block_m) *block_m = v.block_m;
  if (block_n) *block_n = v.block_n;
  if (waves) *waves = v.waves;
  if (stages) *stages = v.stages;
  if (key_split) *key_split = v.key_split;
  if (soft_exp) *soft_exp = v.soft_exp;
  return ATTN_OK;
}

const char* attn_strerror(int status) {
  switch (status) {
    case ATTN_OK: return "success";
    case ATTN_ERR_NULL: return "null pointer";
    case ATTN_ERR_DTYPE: return "unsupported dtype";
    case ATTN_ERR_SHAPE: return "unsupported or invalid shape";
    case ATTN_ERR_ALIGN: return "misaligned pointer";
    case ATTN_ERR_SCALE: return "scale is not finite";
    case ATTN_ERR_DEVICE: return "no gfx950 device";
    case ATTN_ERR_LAUNCH: return "kernel launch failed";
    case ATTN_ERR_ARG: return "invalid option";
    case ATTN_ERR_SCRATCH: return "problem needs more than the static scratch";
    default: return "unknown status";
  }
}

const char* attn_last_error(void) { return g_last_error; }

}  // extern "C"
