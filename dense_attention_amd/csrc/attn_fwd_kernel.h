// Fused dense attention forward for gfx950 (MI355X): device code.
//
// One workgroup processes work items (batch, head, query tile) in a persistent
// loop; inside an item it holds its Q rows in registers and streams the K/V
// tiles of the head through a double-buffered LDS ring, computing
//   S = Q·Kᵀ on MFMA, an online softmax in base 2, and O += P·V on MFMA,
// then O / rowsum and the natural-log LSE.  This is the loop of "B200
// Attention Kernel from Scratch to Near-SOTA in 60 Diagrams", Chapter 1 ("ii.
// Work Parallelization", sections A-C), mapped onto CDNA4 wave64 MFMA.
//
// Register layout (v_mfma_f32_32x32x16_{bf16,f16}; lane = 32·hh + lr):
//   * the kernel computes Sᵀ = K·Qᵀ, so a lane owns one query (column lr) and
//     its accumulator entry i of a 32-key block holds key 16·hh + i.  For that
//     the A-operand lane with MFMA row r reads key lane_key(r).
//   * O is accumulated transposed, Oᵀ = Vᵀ·Pᵀ: the P fragment is the Sᵀ
//     accumulator itself (rounded to 16 bits, never through LDS), and the
//     A-operand row r holds head-dim index lane_key(r), so accumulator i of a
//     32-wide head-dim block holds d = 16·hh + i of the lane's query.
//   * a row max needs one exchange between lanes l and l^32
//     (v_permlane32_swap); row sums stay lane-partial until the epilogue.
//
// Memory path: K and V tiles go from HBM straight into LDS
// (global_load_lds_dwordx4: lane i of a wave writes 16 bytes at base + 16·i,
// so the LDS placement of every 16-byte chunk is chosen through the global
// address each lane loads).  LDS rows are padded (K: +16 bytes, V: +64 bytes)
// so that every LDS read is a per-lane base plus an immediate offset and no
// two lanes of a 64-bank pass hit the same bank:
//   * K rows are stored in MFMA-lane order (LDS row p of a 32-row block holds
//     key lane_key(p)); the A operand of Sᵀ is one ds_read_b128 per lane;
//   * V rows are stored in key order; the A operand of Oᵀ comes from two
//     ds_read_b64_tr_b16, whose 16-lane transpose turns four 8-byte row pieces
//     into four key-contiguous columns.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace attn {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
typedef _Float16 f16x8_t __attribute__((ext_vector_type(8)));
typedef _Float16 f16x2_t __attribute__((ext_vector_type(2)));
typedef float f32x16_t __attribute__((ext_vector_type(16)));
typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2_t __attribute__((ext_vector_type(2)));
typedef short i16x4_t __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) char lds_t;

struct BF16 {};
struct F16 {};

template <typename T>
struct Mma;

template <>
struct Mma<BF16> {
  static __device__ __forceinline__ f32x16_t mfma(u32x4_t a, u32x4_t b, f32x16_t c) {
    return __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8_t, a),
                                                   __builtin_bit_cast(bf16x8_t, b), c, 0, 0, 0);
  }
  // Round two fp32 values to bf16 (nearest-even) and pack them, lo first.
  static __device__ __forceinline__ uint32_t pack(float lo, float hi) {
    bf16x2_t r = {(__bf16)lo, (__bf16)hi};
    return __builtin_bit_cast(uint32_t, r);
  }
};

template <>
struct Mma<F16> {
  static __device__ __forceinline__ f32x16_t mfma(u32x4_t a, u32x4_t b, f32x16_t c) {
    return __builtin_amdgcn_mfma_f32_32x32x16_f16(__builtin_bit_cast(f16x8_t, a),
                                                  __builtin_bit_cast(f16x8_t, b), c, 0, 0, 0);
  }
  static __device__ __forceinline__ uint32_t pack(float lo, float hi) {
    f16x2_t r = {(_Float16)lo, (_Float16)hi};
    return __builtin_bit_cast(uint32_t, r);
  }
};

// Kernel arguments (by value).
struct Params {
  const uint16_t* q;
  const uint16_t* k;
  const uint16_t* v;
  uint16_t* o;
  float* lse;        // may be null
  int S;             // sequence length
  int n_qtiles;      // ceil(S / BM)
  int n_items;       // B * H * n_qtiles
  int xcd_remap;     // 1: the grid is a multiple of 8, group items per XCD
  float c;           // scale * log2(e): scores in log2 units are s * c
  float thr;         // lazy-rescale threshold (log2 units)
};

// MFMA row r of a 32-row block -> row of the K tile (or head-dim index of the
// V tile) it reads, chosen so that accumulator entry i of lane half hh lands
// on row 16·hh + i.  Aligned groups of 4 rows map to 4 consecutive rows.
__device__ __forceinline__ int lane_key(int r) {
  return (((r >> 2) & 1) << 4) | ((r >> 3) << 2) | (r & 3);
}
template <int D_, int BN_, int NW_, int QB_>
struct Tile {
  static constexpr int D = D_;
  static constexpr int BN = BN_;            // keys per K/V tile
  static constexpr int NW = NW_;            // waves per workgroup
  static constexpr int QB = QB_;            // 32-query blocks per wave
  static constexpr int NT = NW * 64;        // threads per workgroup
  static constexpr int BM = NW * QB * 32;   // query rows per work item
  static constexpr int DC = D / 8;          // 16-byte chunks per row
  static constexpr int KS = D * 2 + 16;     // LDS row stride of K (bytes)
  static constexpr int VS = D * 2 + 64;     // LDS row stride of V (bytes)
  static constexpr int K_TILE = BN * KS;
  static constexpr int V_TILE = BN * VS;
  static constexpr int STAGE_BYTES = K_TILE + V_TILE;
  static constexpr int STAGES = 2;
  static constexpr int LDS_BYTES = STAGES * STAGE_BYTES;
  // Waves per SIMD the register allocation targets.
  static constexpr int WPE = NW / 4;
  static_assert(BN % 32 == 0 && D % 32 == 0, "tile sizes");
  static_assert(K_TILE % 1024 == 0 && V_TILE % 1024 == 0, "tiles must be whole DMA blocks");
};

// One 16-byte HBM -> LDS copy per lane (global_load_lds_dwordx4); the LDS
// destination `dst` is wave-uniform and lane i writes dst + 16·i.  Kept as a
// non-template function: the host compilation pass rejects the builtin inside
// implicitly instantiated templates.
__device__ __forceinline__ void dma16(const uint16_t* src, lds_t* dst) {
  __builtin_amdgcn_global_load_lds(src, (__attribute__((address_space(3))) void*)dst, 16, 0, 0);
}

// Issue the HBM -> LDS copy of rows kb .. kb+BN-1 of one head's K or V into a
// padded tile of row stride STRIDE.  With LANE_ORDER, LDS row p of each
// 32-row block receives key lane_key(p).  Rows past S are clamped to row S-1
// (their scores are masked and their P is 0).  Pad slots are not loaded.
template <class TL, int STRIDE, bool LANE_ORDER>
__device__ __forceinline__ void dma_tile(const uint16_t* __restrict__ src, int kb, int S,
                                         lds_t* dst, int wave, int lane) {
  constexpr int SPR = STRIDE / 16;                  // 16-byte slots per LDS row
  constexpr int BLOCKS = TL::BN * SPR / 64;         // 1 KiB blocks per tile
  constexpr int BPW = (BLOCKS + TL::NW - 1) / TL::NW;
#pragma unroll
  for (int t = 0; t < BPW; ++t) {
    const int blk = wave * BPW + t;
    if (BLOCKS % TL::NW == 0 || blk < BLOCKS) {
      const int slot = blk * 64 + lane;
      const int p = slot / SPR;
      const int c = slot - p * SPR;
      if (c < TL::DC) {
        const int key = LANE_ORDER ? ((p & ~31) | lane_key(p & 31)) : p;
        const int grow = min(kb + key, S - 1);
        dma16(src + (size_t)grow * TL::D + c * 8, dst + blk * 1024);
      }
    }
  }
}

__device__ __forceinline__ void wait_vmem() {
  // s_waitcnt vmcnt(0) (expcnt and lgkmcnt left at their maxima).
  __builtin_amdgcn_s_waitcnt(0x0F70);
}

__device__ __forceinline__ u32x4_t ld_global16(const uint16_t* p) {
  return *reinterpret_cast<const u32x4_t*>(p);
}

__device__ __forceinline__ u32x4_t ld_lds16(const lds_t* p) {
  return *reinterpret_cast<const __attribute__((address_space(3))) u32x4_t*>(p);
}

__device__ __forceinline__ u32x2_t ld_lds_tr(const lds_t* p) {
  i16x4_t r = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
      (__attribute__((address_space(3))) i16x4_t*)(p));
  return __builtin_bit_cast(u32x2_t, r);
}

__device__ __forceinline__ float lane_pair_max(float x) {
  auto r = __builtin_amdgcn_permlane32_swap(__builtin_bit_cast(uint32_t, x),
                                            __builtin_bit_cast(uint32_t, x), false, false);
  return fmaxf(__builtin_bit_cast(float, (uint32_t)r[0]), __builtin_bit_cast(float, (uint32_t)r[1]));
}
__device__ __forceinline__ float lane_pair_min(float x) {
  auto r = __builtin_amdgcn_permlane32_swap(__builtin_bit_cast(uint32_t, x),
                                            __builtin_bit_cast(uint32_t, x), false, false);
  return fminf(__builtin_bit_cast(float, (uint32_t)r[0]), __builtin_bit_cast(float, (uint32_t)r[1]));
}
__device__ __forceinline__ float lane_pair_sum(float x) {
  auto r = __builtin_amdgcn_permlane32_swap(__builtin_bit_cast(uint32_t, x),
                                            __builtin_bit_cast(uint32_t, x), false, false);
  return __builtin_bit_cast(float, (uint32_t)r[0]) + __builtin_bit_cast(float, (uint32_t)r[1]);
}

// Per-wave state of one work item.
template <class TL>
struct WaveState {
  u32x4_t qf[TL::QB][TL::D / 16];        // Q fragments (B operand of Sᵀ)
  f32x16_t o[TL::QB][TL::D / 32];        // Oᵀ accumulators
  float m[TL::QB];                       // kept row maximum, log2 units
  float l[TL::QB];                       // lane-partial row sum relative to m
};

// One K/V tile: Sᵀ = K·Qᵀ, online softmax, Oᵀ += Vᵀ·Pᵀ.  MASK handles a
// partial last tile (keys >= S get probability 0).  NEG is set when the score
// multiplier c is negative: the largest c·s is then c·min(s).
template <class T, class TL, bool MASK, bool NEG>
__device__ __forceinline__ void tile_step(WaveState<TL>& ws, const lds_t* kl, const lds_t* vl,
                                          int kb, int S, float c, float thr, int lane) {
  constexpr int D = TL::D, BN = TL::BN, QB = TL::QB, NB = BN / 32, DB = D / 32, DT = D / 16;
  const int lr = lane & 31;
  const int hh = lane >> 5;
  const lds_t* kbase_l = kl + lr * TL::KS + hh * 16;

  // ---- Sᵀ = K · Qᵀ ----------------------------------------------------------
  f32x16_t sacc[QB][NB];
#pragma unroll
  for (int qb = 0; qb < QB; ++qb)
#pragma unroll
    for (int nb = 0; nb < NB; ++nb)
#pragma unroll
      for (int i = 0; i < 16; ++i) sacc[qb][nb][i] = 0.f;
#pragma unroll
  for (int nb = 0; nb < NB; ++nb) {
#pragma unroll
    for (int t = 0; t < DT; ++t) {
      const u32x4_t a = ld_lds16(kbase_l + nb * 32 * TL::KS + t * 32);
#pragma unroll
      for (int qb = 0; qb < QB; ++qb) sacc[qb][nb] = Mma<T>::mfma(a, ws.qf[qb][t], sacc[qb][nb]);
    }
  }

  // ---- online softmax (base 2, lazy rescale) --------------------------------
  const int kbase = kb + 16 * hh;  // key of accumulator entry 0 of block 0
  constexpr float kInit = NEG ? __builtin_inff() : -__builtin_inff();
  uint32_t pk[QB][NB][8];
#pragma unroll
  for (int qb = 0; qb < QB; ++qb) {
    float m4[4] = {kInit, kInit, kInit, kInit};
#pragma unroll
    for (int nb = 0; nb < NB; ++nb)
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        float s = sacc[qb][nb][i];
        if (MASK && kbase + nb * 32 + i >= S) s = kInit;
        m4[i & 3] = NEG ? fminf(m4[i & 3], s) : fmaxf(m4[i & 3], s);
      }
    float mx;
    if (NEG)
      mx = lane_pair_min(fminf(fminf(m4[0], m4[1]), fminf(m4[2], m4[3])));
    else
      mx = lane_pair_max(fmaxf(fmaxf(m4[0], m4[1]), fmaxf(m4[2], m4[3])));
  const float mcand = mx * c;  // tile row maximum in log2 units
    const float mold = ws.m[qb];
    const bool rebase = (mold == -__builtin_inff()) || (mcand > mold + thr);
    const float mnew = rebase ? mcand : mold;
    if (__builtin_amdgcn_ballot_w64(rebase) != 0) {
      const float alpha = __builtin_amdgcn_exp2f(mold - mnew);  // 0 on the first tile
      ws.l[qb] *= alpha;
#pragma unroll
      for (int db = 0; db < DB; ++db)
#pragma unroll
        for (int i = 0; i < 16; ++i) ws.o[qb][db][i] *= alpha;
    }
    ws.m[qb] = mnew;
    const float nm = -mnew;
    float ls[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int nb = 0; nb < NB; ++nb) {
      float pv[16];
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        float e = __builtin_amdgcn_exp2f(__builtin_fmaf(sacc[qb][nb][i], c, nm));
        if (MASK && kbase + nb * 32 + i >= S) e = 0.f;
        pv[i] = e;
        ls[i & 3] += e;
      }
#pragma unroll
      for (int i = 0; i < 8; ++i) pk[qb][nb][i] = Mma<T>::pack(pv[2 * i], pv[2 * i + 1]);
    }
    ws.l[qb] += (ls[0] + ls[1]) + (ls[2] + ls[3]);
  }

  // ---- Oᵀ += Vᵀ · Pᵀ ----------------------------------------------------------
  // Transpose-read geometry: lane group g = lane/16 covers key half h = g/2 and
  // head-dim half gp = g%2; inside the group, lane i reads key row i/4 and the
  // 8-byte piece of head-dim columns chosen so that the result is lane_key-ordered.
  const int g = lane >> 4;
  const int li = lane & 15;
  const lds_t* vbase_l = vl + (16 * (g >> 1) + (li >> 2)) * TL::VS +
                         (2 * (li & 1) + (g & 1)) * 16 + ((li >> 1) & 1) * 8;
#pragma unroll
  for (int nb = 0; nb < NB; ++nb) {
#pragma unroll
    for (int mm = 0; mm < 2; ++mm) {
#pragma unroll
      for (int db = 0; db < DB; ++db) {
        const lds_t* pv0 = vbase_l + (nb * 32 + 8 * mm) * TL::VS + db * 64;
        const u32x2_t lo = ld_lds_tr(pv0);
        const u32x2_t hi = ld_lds_tr(pv0 + 4 * TL::VS);
        const u32x4_t a = {lo[0], lo[1], hi[0], hi[1]};
#pragma unroll
        for (int qb = 0; qb < QB; ++qb) {
          const u32x4_t b = {pk[qb][nb][4 * mm + 0], pk[qb][nb][4 * mm + 1],
                             pk[qb][nb][4 * mm + 2], pk[qb][nb][4 * mm + 3]};
          ws.o[qb][db] = Mma<T>::mfma(a, b, ws.o[qb][db]);
        }
      }
    }
  }
}

template <class T, class TL, bool NEG>
__device__ __forceinline__ void process_item(const Params& p, lds_t* smem, int item, int wave,
                                             int lane) {
  constexpr int D = TL::D, BN = TL::BN, QB = TL::QB, DB = D / 32, DT = D / 16;
  const int lr = lane & 31;
  const int hh = lane >> 5;
  const int S = p.S;

  const int bh = item / p.n_qtiles;
  const int qt = item - bh * p.n_qtiles;
  const size_t head = (size_t)bh * (size_t)S * D;
  const uint16_t* __restrict__ qh = p.q + head;
  const uint16_t* __restrict__ kh = p.k + head;
  const uint16_t* __restrict__ vh = p.v + head;

  const int nt = (S + BN - 1) / BN;

  // Start the first K/V tile, then load Q while it flies.
  dma_tile<TL, TL::KS, true>(kh, 0, S, smem, wave, lane);
  dma_tile<TL, TL::VS, false>(vh, 0, S, smem + TL::K_TILE, wave, lane);

  WaveState<TL> ws;
#pragma unroll
  for (int qb = 0; qb < QB; ++qb) {
    const int row = qt * TL::BM + (wave * QB + qb) * 32 + lr;
#pragma unroll
    for (int t = 0; t < DT; ++t) {
      u32x4_t x = {0u, 0u, 0u, 0u};
      if (row < S) x = ld_global16(qh + (size_t)row * D + 16 * t + 8 * hh);
      ws.qf[qb][t] = x;
    }
    ws.m[qb] = -__builtin_inff();
    ws.l[qb] = 0.f;
#pragma unroll
    for (int db = 0; db < DB; ++db)
#pragma unroll
      for (int i = 0; i < 16; ++i) ws.o[qb][db][i] = 0.f;
  }
  wait_vmem();
  __syncthreads();

  // Full tiles.  The copy of tile j+1 is issued before tile j is computed and
  // waited for after it.
  const int nfull = S / BN;
  for (int j = 0; j < nfull; ++j) {
    const lds_t* kl = smem + (j & 1) * TL::STAGE_BYTES;
    if (j + 1 < nt) {
      lds_t* nk = smem + ((j + 1) & 1) * TL::STAGE_BYTES;
      dma_tile<TL, TL::KS, true>(kh, (j + 1) * BN, S, nk, wave, lane);
      dma_tile<TL, TL::VS, false>(vh, (j + 1) * BN, S, nk + TL::K_TILE, wave, lane);
    }
    tile_step<T, TL, false, NEG>(ws, kl, kl + TL::K_TILE, j * BN, S, p.c, p.thr, lane);
    wait_vmem();
    __syncthreads();
  }
  // Partial last tile (S not a multiple of BN), with keys >= S masked.
  if (nfull < nt) {
    const lds_t* kl = smem + (nfull & 1) * TL::STAGE_BYTES;
    tile_step<T, TL, true, NEG>(ws, kl, kl + TL::K_TILE, nfull * BN, S, p.c, p.thr, lane);
    __syncthreads();
  }

  // ---- epilogue: O / l, round, store; LSE ------------------------------------
#pragma unroll
  for (int qb = 0; qb < QB; ++qb) {
    const float lt = lane_pair_sum(ws.l[qb]);
    const int row = qt * TL::BM + (wave * QB + qb) * 32 + lr;
    if (row < S) {
      const float inv = 1.0f / lt;
      uint16_t* orow = p.o + head + (size_t)row * D;
#pragma unroll
      for (int db = 0; db < DB; ++db) {
        uint32_t w[8];
#pragma unroll
        for (int i = 0; i < 8; ++i)
          w[i] = Mma<T>::pack(ws.o[qb][db][2 * i] * inv, ws.o[qb][db][2 * i + 1] * inv);
        u32x4_t w0 = {w[0], w[1], w[2], w[3]};
        u32x4_t w1 = {w[4], w[5], w[6], w[7]};
        *reinterpret_cast<u32x4_t*>(orow + db * 32 + 16 * hh) = w0;
        *reinterpret_cast<u32x4_t*>(orow + db * 32 + 16 * hh + 8) = w1;
      }
      if (p.lse != nullptr && hh == 0) {
        // ln(sum_j exp(s_j * scale)) = (m + log2(l)) * ln 2
        p.lse[(size_t)bh * S + row] = (ws.m[qb] + __builtin_amdgcn_logf(lt)) * 0.69314718055994531f;
      }
    }
  }
}

template <class T, class TL, bool NEG>
__global__ __launch_bounds__(TL::NT) __attribute__((amdgpu_waves_per_eu(TL::WPE, TL::WPE)))
void attn_fwd_kernel(Params p) {
  __shared__ __attribute__((aligned(1024))) char smem_raw[TL::LDS_BYTES];
  lds_t* smem = (lds_t*)smem_raw;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int lane = threadIdx.x & 63;
  const int G = gridDim.x;
  // Persistent loop over work items ("B200 Attention Kernel from Scratch to
  // Near-SOTA in 60 Diagrams", Chapter 14 - Persistent: a static grid-stride
  // assignment).  Workgroups are dispatched round-robin over the 8 XCDs, so
  // with xcd_remap the items of one round are renumbered to give each XCD a
  // contiguous run of items, i.e. the query tiles of the same heads, whose
  // K/V then stay in that XCD's L2.
  for (int round = 0;; ++round) {
    const int base = round * G;
    if (base >= p.n_items) break;
    int item = base + (int)blockIdx.x;
    if (p.xcd_remap) item = base + (int)(blockIdx.x & 7) * (G >> 3) + (int)(blockIdx.x >> 3);
    if (item < p.n_items) process_item<T, TL, NEG>(p, smem, item, wave, lane);
  }
}

}  // namespace attn
