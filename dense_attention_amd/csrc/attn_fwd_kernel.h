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
//     A operand reads Vᵀ rows (head-dim index) lane_key(r), so accumulator i
//     of a 32-wide head-dim block holds d = 16·hh + i of the lane's query.
//   * a row max needs one exchange between lanes l and l^32
//     (v_permlane32_swap); row sums stay lane-partial until the epilogue.
//
// LDS layout per ring stage: K tile [BN][D] and Vᵀ tile [D][BN] (keys
// contiguous), both with 16-byte chunks XOR-swizzled by row_swizzle(row) so
// that each group of 8 consecutive lanes of a ds_read_b128 hits 8 distinct
// chunk slots.
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

// MFMA row r of a 32-row block -> row of the K (or Vᵀ) tile it reads, chosen
// so that accumulator entry i of lane half hh lands on row 16·hh + i.
__device__ __forceinline__ int lane_key(int r) {
  return (((r >> 2) & 1) << 4) | ((r >> 3) << 2) | (r & 3);
}
// Inverse of lane_key on [0, 32).
__device__ __forceinline__ int key_lane(int x) {
  return (((x >> 2) & 3) << 3) | (((x >> 4) & 1) << 2) | (x & 3);
}
// XOR applied to the 16-byte chunk index of LDS row `row`; `mask` = chunks per row - 1.
__device__ __forceinline__ int row_swizzle(int row, int mask) {
  return key_lane(row & 31) & mask;
}

__device__ __forceinline__ u32x4_t ld_global16(const uint16_t* p) {
  return *reinterpret_cast<const u32x4_t*>(p);
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

template <int D_, int BN_, int NW_, int QB_>
struct Tile {
  static constexpr int D = D_;
  static constexpr int BN = BN_;            // keys per K/V tile
  static constexpr int NW = NW_;            // waves per workgroup
  static constexpr int QB = QB_;            // 32-query blocks per wave
  static constexpr int NT = NW * 64;        // threads per workgroup
  static constexpr int BM = NW * QB * 32;   // query rows per work item
  static constexpr int DC = D / 8;          // 16-byte chunks per K row
  static constexpr int VC = BN / 8;         // 16-byte chunks per Vᵀ row
  static constexpr int KCH = BN * DC;       // 16-byte chunks per K tile
  static constexpr int KPT = (KCH + NT - 1) / NT;
  // Vᵀ staging unit: UK consecutive keys × 8 head-dim entries per thread.
  static constexpr int UK = ((BN / 8) * DC >= NT) ? 8 : 4;
  static constexpr int NU = (BN / UK) * DC;
  static constexpr int UPT = (NU + NT - 1) / NT;
  static constexpr int K_BYTES = BN * D * 2;
  static constexpr int V_BYTES = D * BN * 2;
  static constexpr int STAGE_BYTES = K_BYTES + V_BYTES;
  static constexpr int STAGES = 2;
  static constexpr int LDS_BYTES = STAGES * STAGE_BYTES;
  // Waves per SIMD the register allocation targets.
  static constexpr int WPE = 1;
  static_assert(BN % 64 == 0, "BN must be a multiple of 64 (Vᵀ rows of >= 128 bytes)");
  static_assert(D % 32 == 0, "D must be a multiple of 32");
};

// Global -> register staging of one K/V tile (rows kb .. kb+BN-1 of one head).
template <class TL>
struct Stage {
  u32x4_t kr[TL::KPT];
  u32x4_t vr[TL::UPT][TL::UK];

  __device__ __forceinline__ void load(const uint16_t* __restrict__ kh,
                                       const uint16_t* __restrict__ vh, int kb, int S, int tid) {
#pragma unroll
    for (int i = 0; i < TL::KPT; ++i) {
      const int idx = tid + i * TL::NT;
      const int key = idx / TL::DC;
      const int c = idx % TL::DC;
      const int row = kb + key;
      u32x4_t x = {0u, 0u, 0u, 0u};
      if ((TL::KCH % TL::NT == 0 || idx < TL::KCH) && row < S)
        x = ld_global16(kh + (size_t)row * TL::D + c * 8);
      kr[i] = x;
    }
#pragma unroll
    for (int i = 0; i < TL::UPT; ++i) {
      const int u = tid + i * TL::NT;
      const int a = u / TL::DC;
      const int c = u % TL::DC;
#pragma unroll
      for (int e = 0; e < TL::UK; ++e) {
        const int row = kb + a * TL::UK + e;
        u32x4_t x = {0u, 0u, 0u, 0u};
        if ((TL::NU % TL::NT == 0 || u < TL::NU) && row < S)
          x = ld_global16(vh + (size_t)row * TL::D + c * 8);
        vr[i][e] = x;
      }
    }
  }

  // Write the staged tile into one LDS ring stage: K as is, V transposed.
  __device__ __forceinline__ void store(char* __restrict__ kl, char* __restrict__ vl, int tid) {
#pragma unroll
    for (int i = 0; i < TL::KPT; ++i) {
      const int idx = tid + i * TL::NT;
      if (TL::KCH % TL::NT == 0 || idx < TL::KCH) {
        const int key = idx / TL::DC;
        const int c = idx % TL::DC;
        const int off = key * (TL::D * 2) + ((c ^ row_swizzle(key, TL::DC - 1)) << 4);
        *reinterpret_cast<u32x4_t*>(kl + off) = kr[i];
      }
    }
#pragma unroll
    for (int i = 0; i < TL::UPT; ++i) {
      const int u = tid + i * TL::NT;
      if (TL::NU % TL::NT == 0 || u < TL::NU) {
        const int a = u / TL::DC;
        const int c = u % TL::DC;
        const int key0 = a * TL::UK;            // first key of the unit within the tile
        const int chunk = key0 >> 3;            // 16-byte chunk of the Vᵀ row
        const int sub = (key0 & 7) * 2;         // byte offset inside the chunk (UK == 4)
#pragma unroll
        for (int dd = 0; dd < 8; ++dd) {
          // Gather element dd of each staged key row: pairs of keys per dword.
          uint32_t w[TL::UK / 2];
#pragma unroll
          for (int e2 = 0; e2 < TL::UK / 2; ++e2) {
            const uint32_t x0 = vr[i][2 * e2][dd >> 1];
            const uint32_t x1 = vr[i][2 * e2 + 1][dd >> 1];
            w[e2] = (dd & 1) ? __builtin_amdgcn_perm(x1, x0, 0x07060302u)
                             : __builtin_amdgcn_perm(x1, x0, 0x05040100u);
          }
          const int d = c * 8 + dd;
          const int off = d * (TL::BN * 2) + ((chunk ^ row_swizzle(d, TL::VC - 1)) << 4) + sub;
          if constexpr (TL::UK == 8) {
            u32x4_t val = {w[0], w[1], w[2], w[3]};
            *reinterpret_cast<u32x4_t*>(vl + off) = val;
          } else {
            u32x2_t val = {w[0], w[1]};
            *reinterpret_cast<u32x2_t*>(vl + off) = val;
          }
        }
      }
    }
  }
};

template <class T, class TL>
__device__ __forceinline__ void process_item(const Params& p, char* __restrict__ smem, int item) {
  constexpr int D = TL::D, BN = TL::BN, QB = TL::QB, NB = BN / 32, DB = D / 32, DT = D / 16;
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int lr = lane & 31;
  const int hh = lane >> 5;
  const int S = p.S;

  const int bh = item / p.n_qtiles;
  const int qt = item - bh * p.n_qtiles;
  const size_t head = (size_t)bh * (size_t)S * D;
  const uint16_t* __restrict__ qh = p.q + head;
  const uint16_t* __restrict__ kh = p.k + head;
  const uint16_t* __restrict__ vh = p.v + head;

  // Q fragments (B operand of Sᵀ = K·Qᵀ): lane holds query lr, head-dim
  // entries 16t + 8hh .. +7 for step t.
  u32x4_t qf[QB][DT];
#pragma unroll
  for (int qb = 0; qb < QB; ++qb) {
    const int row = qt * TL::BM + (wave * QB + qb) * 32 + lr;
#pragma unroll
    for (int t = 0; t < DT; ++t) {
      u32x4_t x = {0u, 0u, 0u, 0u};
      if (row < S) x = ld_global16(qh + (size_t)row * D + 16 * t + 8 * hh);
      qf[qb][t] = x;
    }
  }

  f32x16_t oacc[QB][DB];
  float m[QB], l[QB];
#pragma unroll
  for (int qb = 0; qb < QB; ++qb) {
    m[qb] = -__builtin_inff();
    l[qb] = 0.f;
#pragma unroll
    for (int db = 0; db < DB; ++db)
#pragma unroll
      for (int i = 0; i < 16; ++i) oacc[qb][db][i] = 0.f;
  }

  const int nt = (S + BN - 1) / BN;
  const float c = p.c;
  const float thr = p.thr;

  Stage<TL> st;
  st.load(kh, vh, 0, S, tid);
  st.store(smem, smem + TL::K_BYTES, tid);
  if (nt > 1) st.load(kh, vh, BN, S, tid);
  __syncthreads();

  // A-operand row this lane reads inside each 32-row block.
  const int arow = lane_key(lr);

  for (int j = 0; j < nt; ++j) {
    const char* __restrict__ kl = smem + (j & 1) * TL::STAGE_BYTES;
    const char* __restrict__ vl = kl + TL::K_BYTES;

    // ---- S^T = K · Q^T -------------------------------------------------
    f32x16_t sacc[QB][NB];
#pragma unroll
    for (int qb = 0; qb < QB; ++qb)
#pragma unroll
      for (int nb = 0; nb < NB; ++nb)
#pragma unroll
        for (int i = 0; i < 16; ++i) sacc[qb][nb][i] = 0.f;

#pragma unroll
    for (int nb = 0; nb < NB; ++nb) {
      const int key = nb * 32 + arow;
      const char* krow = kl + key * (D * 2);
      const int sw = row_swizzle(key, TL::DC - 1);
#pragma unroll
      for (int t = 0; t < DT; ++t) {
        const u32x4_t a = *reinterpret_cast<const u32x4_t*>(krow + (((2 * t + hh) ^ sw) << 4));
#pragma unroll
        for (int qb = 0; qb < QB; ++qb) sacc[qb][nb] = Mma<T>::mfma(a, qf[qb][t], sacc[qb][nb]);
      }
    }

    // ---- online softmax (base 2, lazy rescale) ---------------------------
    const bool tail = (j == nt - 1) && (S % BN != 0);
    const int kbase = j * BN + 16 * hh;  // key of accumulator entry 0 of block 0
    uint32_t pk[QB][NB][8];
#pragma unroll
    for (int qb = 0; qb < QB; ++qb) {
      float mx;
      if (c >= 0.f) {
        mx = -__builtin_inff();
#pragma unroll
        for (int nb = 0; nb < NB; ++nb)
#pragma unroll
          for (int i = 0; i < 16; ++i) {
            float s = sacc[qb][nb][i];
            if (tail && kbase + nb * 32 + i >= S) s = -__builtin_inff();
            mx = fmaxf(mx, s);
          }
        mx = lane_pair_max(mx);
      } else {
        mx = __builtin_inff();
#pragma unroll
        for (int nb = 0; nb < NB; ++nb)
#pragma unroll
          for (int i = 0; i < 16; ++i) {
            float s = sacc[qb][nb][i];
            if (tail && kbase + nb * 32 + i >= S) s = __builtin_inff();
            mx = fminf(mx, s);
          }
        mx = lane_pair_min(mx);
      }
      const float mcand = mx * c;  // tile row maximum in log2 units
      const float mold = m[qb];
      const bool rebase = (mold == -__builtin_inff()) || (mcand > mold + thr);
      const float mnew = rebase ? mcand : mold;
      if (__builtin_amdgcn_ballot_w64(rebase) != 0) {
        const float alpha = __builtin_amdgcn_exp2f(mold - mnew);  // 0 on the first tile
        l[qb] *= alpha;
#pragma unroll
        for (int db = 0; db < DB; ++db)
#pragma unroll
          for (int i = 0; i < 16; ++i) oacc[qb][db][i] *= alpha;
      }
      m[qb] = mnew;
      const float nm = -mnew;
      float ls = 0.f;
#pragma unroll
      for (int nb = 0; nb < NB; ++nb) {
        float pv[16];
#pragma unroll
        for (int i = 0; i < 16; ++i) {
          float e = __builtin_amdgcn_exp2f(__builtin_fmaf(sacc[qb][nb][i], c, nm));
          if (tail && kbase + nb * 32 + i >= S) e = 0.f;
          pv[i] = e;
          ls += e;
        }
#pragma unroll
        for (int i = 0; i < 8; ++i) pk[qb][nb][i] = Mma<T>::pack(pv[2 * i], pv[2 * i + 1]);
      }
      l[qb] += ls;
    }

    // ---- O^T += V^T · P^T --------------------------------------------------
#pragma unroll
    for (int nb = 0; nb < NB; ++nb) {
#pragma unroll
      for (int mm = 0; mm < 2; ++mm) {
        const int chunk = nb * 4 + 2 * hh + mm;
#pragma unroll
        for (int db = 0; db < DB; ++db) {
          const int d = db * 32 + arow;
          const u32x4_t a = *reinterpret_cast<const u32x4_t*>(
              vl + d * (BN * 2) + ((chunk ^ row_swizzle(d, TL::VC - 1)) << 4));
#pragma unroll
          for (int qb = 0; qb < QB; ++qb) {
            const u32x4_t b = {pk[qb][nb][4 * mm + 0], pk[qb][nb][4 * mm + 1],
                               pk[qb][nb][4 * mm + 2], pk[qb][nb][4 * mm + 3]};
            oacc[qb][db] = Mma<T>::mfma(a, b, oacc[qb][db]);
          }
        }
      }
    }

    // ---- refill the ring -------------------------------------------------
    if (j + 1 < nt) {
      char* ks = smem + ((j + 1) & 1) * TL::STAGE_BYTES;
      st.store(ks, ks + TL::K_BYTES, tid);
    }
    if (j + 2 < nt) st.load(kh, vh, (j + 2) * BN, S, tid);
    __syncthreads();
  }

  // ---- epilogue: O / l, round, store; LSE -------------------------------------
#pragma unroll
  for (int qb = 0; qb < QB; ++qb) {
    const float lt = lane_pair_sum(l[qb]);
    const int row = qt * TL::BM + (wave * QB + qb) * 32 + lr;
    if (row < S) {
      const float inv = 1.0f / lt;
      uint16_t* orow = p.o + head + (size_t)row * D;
#pragma unroll
      for (int db = 0; db < DB; ++db) {
        uint32_t w[8];
#pragma unroll
        for (int i = 0; i < 8; ++i)
          w[i] = Mma<T>::pack(oacc[qb][db][2 * i] * inv, oacc[qb][db][2 * i + 1] * inv);
        u32x4_t w0 = {w[0], w[1], w[2], w[3]};
        u32x4_t w1 = {w[4], w[5], w[6], w[7]};
        *reinterpret_cast<u32x4_t*>(orow + db * 32 + 16 * hh) = w0;
        *reinterpret_cast<u32x4_t*>(orow + db * 32 + 16 * hh + 8) = w1;
      }
      if (p.lse != nullptr && hh == 0) {
        // ln(sum_j exp(s_j * scale)) = (m + log2(l)) * ln 2
        p.lse[(size_t)bh * S + row] = (m[qb] + __builtin_amdgcn_logf(lt)) * 0.69314718055994531f;
      }
    }
  }
}

template <class T, class TL>
__global__ __launch_bounds__(TL::NT) __attribute__((amdgpu_waves_per_eu(TL::WPE, TL::WPE))) void attn_fwd_kernel(Params p) {
  __shared__ __attribute__((aligned(16))) char smem[TL::LDS_BYTES];
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
    if (item < p.n_items) process_item<T, TL>(p, smem, item);
  }
}

}  // namespace attn
