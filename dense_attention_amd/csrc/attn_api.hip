// C ABI of the fused dense attention forward (declared in include/attn.h):
// argument validation, tile-variant choice, persistent-grid sizing and the
// launch on the caller's stream.  No allocation, no synchronisation.
#include <hip/hip_runtime.h>

#include <cmath>
#include <cstdint>
#include <cstdio>
#include <cstring>
#include <mutex>

#include "attn.h"
#include "attn_fwd_kernel.h"

namespace {

using attn::BF16;
using attn::F16;
using attn::Params;
using attn::Tile;

constexpr float kDefaultThreshold = 8.0f;  // log2 units
constexpr float kLog2e = 1.4426950408889634f;

thread_local char g_last_error[256] = "";

int fail(int status, const char* detail) {
  std::snprintf(g_last_error, sizeof(g_last_error), "%s", detail ? detail : "");
  return status;
}

typedef hipError_t (*launch_fn)(const Params&, bool neg, int grid, hipStream_t stream);
typedef hipError_t (*occ_fn)(int* blocks_per_cu);

// Negative score multipliers use a separate instantiation (the running
// maximum of c·s is then taken over min(s)).
template <class T, class TL>
hipError_t launch_impl(const Params& p, bool neg, int grid, hipStream_t stream) {
  if (neg)
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
  launch_fn launch;
  occ_fn occupancy;
};

template <class T, int DTYPE, class TL>
constexpr Variant make_variant(int id) {
  return Variant{id, DTYPE, TL::D, TL::BM, TL::BN, TL::NW, TL::STAGES, TL::LDS_BYTES,
                 &launch_impl<T, TL>, &occupancy_impl<T, TL>};
}

// Tile variants: ids are stable; the first matching entry for (D, dtype) in
// kDefaults is the library's choice.
const Variant kVariants[] = {
    make_variant<BF16, ATTN_BF16, Tile<128, 64, 8, 1>>(1),
    make_variant<F16, ATTN_F16, Tile<128, 64, 8, 1>>(2),
    make_variant<BF16, ATTN_BF16, Tile<64, 64, 4, 1>>(3),
    make_variant<F16, ATTN_F16, Tile<64, 64, 4, 1>>(4),
    make_variant<BF16, ATTN_BF16, Tile<128, 64, 4, 1>>(5),
    make_variant<F16, ATTN_F16, Tile<128, 64, 4, 1>>(6),
    make_variant<BF16, ATTN_BF16, Tile<64, 64, 8, 1>>(7),
    make_variant<F16, ATTN_F16, Tile<64, 64, 8, 1>>(8),
    make_variant<BF16, ATTN_BF16, Tile<128, 128, 4, 1>>(9),
    make_variant<F16, ATTN_F16, Tile<128, 128, 4, 1>>(10),
    make_variant<BF16, ATTN_BF16, Tile<128, 64, 4, 2>>(11),
    make_variant<F16, ATTN_F16, Tile<128, 64, 4, 2>>(12),
};
constexpr int kNumVariants = sizeof(kVariants) / sizeof(kVariants[0]);

const Variant* find_variant(int id) {
  for (int i = 0; i < kNumVariants; ++i)
    if (kVariants[i].id == id) return &kVariants[i];
  return nullptr;
}

const Variant* default_variant(int D, int dtype) {
  for (int i = 0; i < kNumVariants; ++i)
    if (kVariants[i].D == D && kVariants[i].dtype == dtype) return &kVariants[i];
  return nullptr;
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
  int n_items = 0;
  int grid = 0;
  int per_cu = 0;
  int num_cus = 0;
  float thr = kDefaultThreshold;
  bool empty = false;
};

// Validation shared by every entry point (data pointers excluded).
int plan_launch(int B, int H, int S, int D, int dtype, float scale,
                const attn_fwd_options_t* opts, bool need_device, Plan* plan) {
  if (dtype != ATTN_F16 && dtype != ATTN_BF16) return fail(ATTN_ERR_DTYPE, "dtype must be ATTN_F16 or ATTN_BF16");
  if (B < 0 || H < 0 || S < 0) return fail(ATTN_ERR_SHAPE, "B, H and S must be >= 0");
  if (D != 64 && D != 128) return fail(ATTN_ERR_SHAPE, "D must be 64 or 128");
  if (!std::isfinite(scale)) return fail(ATTN_ERR_SCALE, "scale must be finite");
  if (opts) {
    for (int r : opts->reserved)
      if (r != 0) return fail(ATTN_ERR_ARG, "reserved option fields must be zero");
    if (opts->grid < 0) return fail(ATTN_ERR_ARG, "grid must be >= 0");
    if (!(opts->rescale_threshold <= 64.0f) && !(opts->rescale_threshold < 0.0f))
      return fail(ATTN_ERR_ARG, "rescale_threshold must be <= 64");
  }
  // 64-bit element offsets are used per head; a single head and the item count
  // must fit in 32-bit indices.
  if ((int64_t)S * D >= (int64_t)1 << 31) return fail(ATTN_ERR_SHAPE, "S*D must be < 2^31");
  if ((int64_t)B * H * (int64_t)S >= (int64_t)1 << 31) return fail(ATTN_ERR_SHAPE, "B*H*S must be < 2^31");

  const Variant* var = default_variant(D, dtype);
  if (opts && opts->variant != 0) {
    var = find_variant(opts->variant);
    if (!var) return fail(ATTN_ERR_ARG, "unknown variant id");
    if (var->D != D || var->dtype != dtype) return fail(ATTN_ERR_ARG, "variant does not support this D/dtype");
  }
  plan->var = var;
  plan->var_index = (int)(var - kVariants);
  plan->thr = (opts && opts->rescale_threshold >= 0.0f) ? opts->rescale_threshold : kDefaultThreshold;
  plan->n_qtiles = (S + var->block_m - 1) / var->block_m;
  plan->n_items = B * H * plan->n_qtiles;
  plan->empty = (plan->n_items == 0);
  if (!need_device) return ATTN_OK;

  const DeviceInfo* di = nullptr;
  int st = device_info(&di);
  if (st != ATTN_OK) return st;
  plan->num_cus = di->num_cus;
  plan->per_cu = di->occupancy[plan->var_index];
  int grid = di->num_cus * plan->per_cu;
  if (opts && opts->grid > 0) grid = opts->grid;
  if (grid > plan->n_items) grid = plan->n_items;
  plan->grid = grid;
  return ATTN_OK;
}

}  // namespace

extern "C" {

int attn_fwd_ex(const void* q, const void* k, const void* v, void* o, float* lse, int B, int H,
                int S, int D, float scale, int dtype, void* stream,
                const attn_fwd_options_t* opts) {
  g_last_error[0] = '\0';
  Plan plan;
  int st = plan_launch(B, H, S, D, dtype, scale, opts, /*need_device=*/false, &plan);
  if (st != ATTN_OK) return st;
  if (plan.empty) return ATTN_OK;
  if (!q || !k || !v || !o) return fail(ATTN_ERR_NULL, "q, k, v and o must be non-null");
  auto misaligned = [](const void* p, uintptr_t a) { return (reinterpret_cast<uintptr_t>(p) & (a - 1)) != 0; };
  if (misaligned(q, 16) || misaligned(k, 16) || misaligned(v, 16) || misaligned(o, 16))
    return fail(ATTN_ERR_ALIGN, "q, k, v and o must be 16-byte aligned");
  if (lse && misaligned(lse, 4)) return fail(ATTN_ERR_ALIGN, "lse must be 4-byte aligned");
  st = plan_launch(B, H, S, D, dtype, scale, opts, /*need_device=*/true, &plan);
  if (st != ATTN_OK) return st;

  Params p;
  p.q = static_cast<const uint16_t*>(q);
  p.k = static_cast<const uint16_t*>(k);
  p.v = static_cast<const uint16_t*>(v);
  p.o = static_cast<uint16_t*>(o);
  p.lse = lse;
  p.S = S;
  p.n_qtiles = plan.n_qtiles;
  p.n_items = plan.n_items;
  p.xcd_remap = (plan.grid % 8 == 0 && plan.grid >= 8) ? 1 : 0;
  p.c = scale * kLog2e;
  p.thr = plan.thr;
  hipError_t e = plan.var->launch(p, p.c < 0.0f, plan.grid, static_cast<hipStream_t>(stream));
  if (e != hipSuccess) return fail(ATTN_ERR_LAUNCH, hipGetErrorString(e));
  return ATTN_OK;
}

int attn_fwd(const void* q, const void* k, const void* v, void* o, float* lse, int B, int H,
             int S, int D, float scale, int dtype, void* stream) {
  return attn_fwd_ex(q, k, v, o, lse, B, H, S, D, scale, dtype, stream, nullptr);
}

int attn_get_config(int B, int H, int S, int D, int dtype, const attn_fwd_options_t* opts,
                    attn_config_t* out) {
  g_last_error[0] = '\0';
  if (!out) return fail(ATTN_ERR_NULL, "out must be non-null");
  Plan plan;
  int st = plan_launch(B, H, S, D, dtype, 1.0f, opts, /*need_device=*/true, &plan);
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
                      int* waves, int* stages) {
  if (index < 0 || index >= kNumVariants) return fail(ATTN_ERR_ARG, "variant index out of range");
  const Variant& v = kVariants[index];
  if (id) *id = v.id;
  if (head_dim) *head_dim = v.D;
  if (dtype) *dtype = v.dtype;
  if (block_m) *block_m = v.block_m;
  if (block_n) *block_n = v.block_n;
  if (waves) *waves = v.waves;
  if (stages) *stages = v.stages;
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
    default: return "unknown status";
  }
}

const char* attn_last_error(void) { return g_last_error; }

}  // extern "C"
