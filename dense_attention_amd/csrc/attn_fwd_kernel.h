// Fused dense attention forward for gfx950 (MI355X): device code.
//
// One workgroup processes work items (batch, head, query tile, key range) in a
// persistent loop; inside an item it holds its Q rows in registers and streams
// the K/V tiles of the head through a two- or three-deep LDS ring, computing
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
// address each lane loads).  LDS rows are padded (K: +16 bytes, V: +64) so
// that every LDS read is a per-lane base plus an immediate offset and no two
// lanes of a 64-bank pass hit the same bank; where padded V rows do not fit,
// V rows are unpadded and swizzled instead (Tile::VSWZ):
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
  // Row sums come from the fp32 p: bf16's rounding (up to 2^-9 relative)
  // would move the LSE of a short or one-key-dominated row by up to 2e-3.
  static constexpr bool PACKED_SUMS = false;
  static __device__ __forceinline__ float sum2(uint32_t, float acc) { return acc; }
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
  // Row sums come from the rounded P itself, one v_dot2c_f32_f16 against
  // (1, 1) per packed pair: half the additions of summing the fp32 p.  fp16
  // rounds P to within 2^-11 relative, which moves a row's LSE by at most
  // 4.9e-4, and O and its normaliser then see the same P.
  static constexpr bool PACKED_SUMS = true;
  static __device__ __forceinline__ float sum2(uint32_t pk, float acc) {
    const f16x2_t one = {(_Float16)1.0f, (_Float16)1.0f};
    return __builtin_amdgcn_fdot2(__builtin_bit_cast(f16x2_t, pk), one, acc, false);
  }
};

// Kernel arguments (by value).  Strides are in elements; the head dimension
// is contiguous.  Work item = (b·H + h, query tile, KV range).
struct Params {
  const uint16_t* q;
  const uint16_t* k;
  const uint16_t* v;
  void* o;               // T elements, or fp32 when o_f32
  float* lse;            // contiguous [.., B, H, Sq]; may be null
  long long q_sb, q_sh;  // batch and head strides
  long long k_sb, k_sh;
  long long v_sb, v_sh;
  long long o_sb, o_sh;
  long long o_split;     // elements between the outputs of consecutive KV ranges
  long long lse_split;
  int q_ss, k_ss, v_ss, o_ss;  // row (token) strides
  int H;
  int BH;                // B * H
  int Sq;                // query rows per head
  int Skv;               // keys per head
  int n_qtiles;          // ceil(Sq / BM)
  int n_splits;          // KV ranges per (head, query tile)
  int split_len;         // keys per range (a multiple of BN; the last may be shorter)
  int n_items;           // B * H * n_qtiles * n_splits
  int xcd_remap;         // 1: the grid is a multiple of 8, group items per XCD
  int o_f32;             // 1: O is stored in fp32, normalised within its KV range
  int coff;              // causal: query row i sees keys j <= i + coff (absolute key index)
  float c;               // scale * log2(e): scores in log2 units are s * c
  float thr;             // lazy-rescale threshold (log2 units)
};

// MFMA row r of a 32-row block -> row of the K tile (or head-dim index of the
// V tile) it reads, chosen so that accumulator entry i of lane half hh lands
// on row 16·hh + i.  Aligned groups of 4 rows map to 4 consecutive rows.
__device__ __forceinline__ int lane_key(int r) {
  return (((r >> 2) & 1) << 4) | ((r >> 3) << 2) | (r & 3);
}
// KSPLIT: the two groups of four waves of an 8-wave workgroup hold the same
// query rows and each streams one half of the item's keys through a K/V ring
// of its own; their partial results are merged through LDS at the end of the
// item.  This keeps two waves on every SIMD (the ping-pong below) with
// 128-row work items, for problems with too few 256-row items to fill the
// device.
// POLY: when > 0, one score in every POLY of a tile gets 2^x from a cubic
// polynomial on the VALU instead of v_exp_f32 (exp2_poly).
template <int D_, int BN_, int NW_, int QB_, bool KSPLIT_ = false, int POLY_ = 0>
struct Tile {
  static constexpr int D = D_;
  static constexpr int BN = BN_;            // keys per K/V tile
  static constexpr int NW = NW_;            // waves per workgroup
  static constexpr int QB = QB_;            // 32-query blocks per wave
  static constexpr bool KSPLIT = KSPLIT_;
  static constexpr int POLY = POLY_;
  static constexpr int GW = KSPLIT ? NW / 2 : NW;  // waves sharing one K/V stream
  static constexpr int NT = NW * 64;        // threads per workgroup
  static constexpr int BM = GW * QB * 32;   // query rows per work item
  static constexpr int DC = D / 8;          // 16-byte chunks per row
  static constexpr int RINGS = KSPLIT ? 2 : 1;
  static constexpr int KS = D * 2 + 16;     // LDS row stride of K (bytes)
  // LDS rows of V: padded by 64 bytes, or, where two-deep rings of padded
  // rows would not fit in LDS (the key split at D = 64 with 128-key tiles),
  // unpadded with bit 2 of the 16-byte chunk index XOR-ed with bit 1 of the
  // row (VSWZ), which keeps the transposed operand reads conflict-free.
  static constexpr bool VSWZ = 2 * RINGS * BN * (KS + D * 2 + 64) > 160 * 1024;
  static constexpr int VS = VSWZ ? D * 2 : D * 2 + 64;
  static constexpr int K_TILE = BN * KS;
  static constexpr int V_TILE = BN * VS;
  // K/V ring depth: three tiles when they fit in LDS, else two.
  static constexpr int STAGES = 3 * RINGS * (BN * (KS + VS)) <= 160 * 1024 ? 3 : 2;
  static constexpr int RING_BYTES = STAGES * (K_TILE + V_TILE);
  // 16-bit O rows leave through LDS where there is room (STAGE_O): each wave
  // writes its rows there in the accumulator layout and reads them back as
  // whole rows, so a store instruction covers a few full rows instead of 32
  // bytes of 32 rows.  The staging area starts at V slot 1, which the next
  // item's first copies (K slots 0-1, V slot 0) never target; its rows are
  // padded by 16 bytes so that the accumulator-layout writes spread over
  // the banks.
  static constexpr int SROW = D * 2 + 16;
  static constexpr int STAGE_OFF = STAGES * K_TILE + V_TILE;
  static constexpr int STAGE_END = STAGE_OFF + NW * QB * 32 * SROW;
  static constexpr bool STAGE_O = !KSPLIT && STAGES == 3 && STAGE_END <= 160 * 1024;
  static constexpr int LDS_BYTES =
      STAGE_O && STAGE_END > RINGS * RING_BYTES ? STAGE_END : RINGS * RING_BYTES;
  // Per-lane 16-byte chunks one wave hands over in the key-split merge: the
  // O accumulators, then (m, l) of each query block.
  static constexpr int XCH = QB * (D / 32) * 4 + 1;
  // Waves per SIMD the register allocation targets.
  static constexpr int WPE = NW / 4;
  // The MFMA phase runs at raised wave priority and the copy blocks of a tile
  // are dealt to the waves round-robin (K blocks first, V blocks continuing
  // where K left off), so every wave issues about as many.  Measured about 1%
  // faster on the shared stream at D = 128, 1-2% on its key split and on the
  // shared stream at D = 64; the key split at D = 64 keeps contiguous blocks
  // (within noise there, and its registers would spill).
  static constexpr bool PRIO = !(KSPLIT && D == 64);
  // D = 64: the Sᵀ and P·V MFMAs of a phase alternate (measured faster there;
  // at D = 128 the split softmax between the P·V MFMAs wins).
  static constexpr bool ALT = D == 64;
  static_assert(BN % 32 == 0 && D % 32 == 0, "tile sizes");
  static_assert(!VSWZ || D == 64, "the V swizzle assumes 128-byte rows");
  static_assert(K_TILE % 1024 == 0 && V_TILE % 1024 == 0, "tiles must be whole DMA blocks");
  static_assert(!KSPLIT || NW == 8, "a key split pairs two groups of four waves");
  static_assert(LDS_BYTES <= 160 * 1024, "LDS");
  static_assert(!KSPLIT || GW * XCH * 1024 <= LDS_BYTES, "merge exchange must fit in the rings");
};

// One 16-byte HBM -> LDS copy per lane (global_load_lds_dwordx4): lane i
// reads base + voff and writes LDS address lds + 16·i; `base` and `lds` are
// wave-uniform.  Written as inline assembly on purpose: the compiler then does
// not track the copy as a pending LDS store, so it does not stall the next LDS
// reads of *other* buffers on it.  Completion is awaited explicitly
// (wait_vmem) before the workgroup barrier that publishes a tile, and no LDS
// location is read while a copy into it is in flight.
__device__ __forceinline__ void dma16(const void* base, uint32_t voff, const lds_t* lds) {
  // Wave-uniform by construction; readfirstlane keeps it in an SGPR where the
  // compiler cannot prove that (it is a no-op on an SGPR value).
  const uint32_t m0v = __builtin_amdgcn_readfirstlane((uint32_t)(uintptr_t)lds);
  asm volatile(
      "s_mov_b32 m0, %2\n\t"
      "s_nop 0\n\t"
      "global_load_lds_dwordx4 %0, %1"
      :
      : "v"(voff), "s"(base), "s"(m0v)
      : "memory", "m0");
}

// HBM -> LDS copy of one K or V tile (rows kb .. kb+BN-1 of one head) into a
// padded LDS tile of row stride STRIDE.  Each of the GW waves that share the
// stream (`wave` is the index among them) owns BPW of the tile's 1 KiB
// blocks; lane i of a block fills 16-byte slot i.  With LANE_ORDER, LDS row p
// of each 32-row block receives key lane_key(p).  Pad slots receive a copy of
// their row's first chunk (never read).  With SWZ (unpadded rows), slot c of
// row p receives chunk c ^ (4·bit 1 of p).  The per-lane byte offsets do not
// depend on the tile, so they are computed once per kernel and a full tile
// costs one address add per block.
template <class TL, int STRIDE, bool LANE_ORDER, int ROT = 0, bool SWZ = false>
struct DmaPlan {
  static constexpr int SPR = STRIDE / 16;              // 16-byte slots per LDS row
  static constexpr int BLOCKS = TL::BN * SPR / 64;     // 1 KiB blocks per tile
  static constexpr int BPW = (BLOCKS + TL::GW - 1) / TL::GW;
  // Block t of wave `wave`: contiguous runs of BPW blocks, or with PRIO dealt
  // round-robin starting at wave ROT.
  __device__ __forceinline__ static int block(int wave, int t) {
    if (TL::PRIO) return (wave + TL::GW - ROT % TL::GW) % TL::GW + t * TL::GW;
    return wave * BPW + t;
  }
  // Byte offset of this lane's chunk from the tile's first row.  Pad slots load
  // chunk 0 of their row again (the pad bytes of an LDS row are never read).
  uint32_t off[BPW];

  __device__ __forceinline__ static void slot_rc(int blk, int lane, int& key, int& c) {
    const int slot = blk * 64 + lane;
    const int p = slot / SPR;
    c = slot - p * SPR;
    if (c >= TL::DC) c = 0;
    if (SWZ) c ^= ((p >> 1) & 1) << 2;
    key = LANE_ORDER ? ((p & ~31) | lane_key(p & 31)) : p;
  }

  // row_bytes: distance of consecutive rows in bytes (BN·row_bytes < 2^31).
  __device__ __forceinline__ void init(int wave, int lane, uint32_t row_bytes) {
#pragma unroll
    for (int t = 0; t < BPW; ++t) {
      int key, c;
      slot_rc(block(wave, t), lane, key, c);
      off[t] = (uint32_t)key * row_bytes + (uint32_t)c * 16u;
    }
  }

  // Full tile whose first row is at `tile`.  `blk < BLOCKS` is wave-uniform.
  __device__ __forceinline__ void issue(const uint16_t* tile, lds_t* dst, int wave) const {
#pragma unroll
    for (int t = 0; t < BPW; ++t) {
      const int blk = block(wave, t);
      if (BLOCKS % TL::GW == 0 || blk < BLOCKS) {
        // Opaque per call: keeps the address as uniform base + 32-bit lane
        // offset instead of a hoisted 64-bit per-lane pointer.
        dma16(tile, off[t], dst + blk * 1024);
      }
    }
  }

  // Tile whose first row is at `tile` and that may run past the last key: its
  // rows at or beyond `rows` are clamped to row rows-1 (their scores are
  // masked and their P is 0).  Rare (last tile of a ragged range), so the
  // lane's row is recomputed here instead of being kept in registers.
  __device__ __forceinline__ void issue_clamped(const uint16_t* tile, int rows, uint32_t row_bytes,
                                                lds_t* dst, int wave, int lane) const {
#pragma unroll
    for (int t = 0; t < BPW; ++t) {
      const int blk = block(wave, t);
      if (BLOCKS % TL::GW == 0 || blk < BLOCKS) {
        int key, c;
        slot_rc(blk, lane, key, c);
        key = min(key, rows - 1);
        dma16(tile, (uint32_t)key * row_bytes + (uint32_t)c * 16u, dst + blk * 1024);
      }
    }
  }
};

__device__ __forceinline__ void wait_vmem() {
  // s_waitcnt vmcnt(0) (expcnt and lgkmcnt left at their maxima).
  __builtin_amdgcn_s_waitcnt(0x0F70);
}

// s_waitcnt vmcnt(N): all but the N most recent vector memory operations of
// the wave have completed (they complete in issue order).
template <int N>
__device__ __forceinline__ void wait_vmem_n() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  __builtin_amdgcn_s_waitcnt(0x0F70 | (N & 15) | ((N >> 4) << 14));
}

__device__ __forceinline__ u32x4_t ld_global16(const uint16_t* p) {
  return *reinterpret_cast<const u32x4_t*>(p);
}

__device__ __forceinline__ u32x4_t ld_lds16(const lds_t* p) {
  return *reinterpret_cast<const __attribute__((address_space(3))) u32x4_t*>(p);
}

__device__ __forceinline__ void st_lds16(lds_t* p, u32x4_t x) {
  *reinterpret_cast<__attribute__((address_space(3))) u32x4_t*>(p) = x;
}

__device__ __forceinline__ u32x2_t ld_lds_tr(const lds_t* p) {
  i16x4_t r = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
      (__attribute__((address_space(3))) i16x4_t*)(p));
  return __builtin_bit_cast(u32x2_t, r);
}

// Bit casts through by-value parameters.  __builtin_bit_cast applied directly
// to an element of an ext_vector_type value (v[i]) reads the vector's first
// element instead; a by-value argument is a plain float or uint32_t.
__device__ __forceinline__ uint32_t f2u(float x) { return __builtin_bit_cast(uint32_t, x); }
__device__ __forceinline__ float u2f(uint32_t x) { return __builtin_bit_cast(float, x); }

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

// A compile-time integer carried through generic lambdas.
template <int V>
struct IntC {
  static constexpr int value = V;
};

// Per-wave state of one work item.
template <class TL>
struct WaveState {
  u32x4_t qf[TL::QB][TL::D / 16];        // Q fragments (B operand of Sᵀ)
  f32x16_t o[TL::QB][TL::D / 32];        // Oᵀ accumulators
  float m[TL::QB];                       // kept row maximum, log2 units
  float l[TL::QB];                       // lane-partial row sum relative to m
};

// ---- register tiles ----------------------------------------------------------------
//
// Sᵀ accumulators of one tile (32 keys per block) and the packed 16-bit P
// fragments made from them (the B operand of Oᵀ += Vᵀ·Pᵀ).

template <class TL>
using SAcc = f32x16_t[TL::QB][TL::BN / 32];
template <class TL>
using PFrag = uint32_t[TL::QB][TL::BN / 32][8];

// 2^x without the transcendental unit: 2^x = 2^n · 2^f with n = floor(x),
// f = x - n in [0, 1), and 2^f from a cubic whose coefficients minimise the
// maximum relative error on [0, 1) with the constant term pinned to 1
// (fit_exp2_poly.py, Remez exchange; max relative error 8.6e-5, below the
// rounding of P to bf16 or fp16).  The selective use of a polynomial for part
// of the exponentials is the B200 page's software exp2 (Chapter 9); the
// coefficients here are fitted independently.  x below -127 is clamped there
// (2^-127 is far below any P that survives the rounding to 16 bits).
__device__ __forceinline__ float exp2_poly(float x) {
  x = fmaxf(x, -127.f);
  // n from floor, not x - fract(x): fract saturates just below 1 for x just
  // below an integer, and x - fract(x) is then not an integer.  f = x - n may
  // round up to 1.0, where the cubic gives 2 - 1.4e-4: still 2^x.
  const float n = __builtin_floorf(x);
  const float f = x - n;
  float p = __builtin_fmaf(0.077067042f, f, 0.227644991f);
  p = __builtin_fmaf(p, f, 0.695116786f);
  p = __builtin_fmaf(p, f, 1.0f);
  return __builtin_amdgcn_ldexpf(p, (int)n);
}

template <class TL>
__device__ __forceinline__ void rescale_o(WaveState<TL>& ws, const float (&alpha)[TL::QB]) {
#pragma unroll
  for (int qb = 0; qb < TL::QB; ++qb)
#pragma unroll
    for (int db = 0; db < TL::D / 32; ++db)
#pragma unroll
      for (int i = 0; i < 16; ++i) ws.o[qb][db][i] *= alpha[qb];
}

// LDS ring: STAGES K buffers then STAGES V buffers; K_t lives in K buffer
// t % STAGES and V_t in V buffer t % STAGES.
template <class TL>
struct Ring {
  lds_t* base;
  __device__ __forceinline__ lds_t* k(int t) const { return base + (t % TL::STAGES) * TL::K_TILE; }
  __device__ __forceinline__ lds_t* v(int t) const {
    return base + TL::STAGES * TL::K_TILE + (t % TL::STAGES) * TL::V_TILE;
  }
};

template <class TL>
struct Copies {
  using KPlan = DmaPlan<TL, TL::KS, true>;
  using VPlan = DmaPlan<TL, TL::VS, false, (TL::BN * TL::KS / 1024) % TL::GW, TL::VSWZ>;
  KPlan k;
  VPlan v;
  // Copy instructions every wave issues for one K tile plus one V tile (at
  // least; waves differ by one where the blocks do not divide evenly).
  static constexpr int MIN_ISSUED = KPlan::BLOCKS / TL::GW + VPlan::BLOCKS / TL::GW;
};

// Epilogue of a work item: O / l (rounded to the output type, or fp32 for a
// partial result over one KV range) and the LSE.  With STAGE_O, 16-bit rows
// go through the wave's own part of the LDS staging area: every ring read of
// the item is over (the item's final barriers), and the next item writes the
// area only after the barrier that starts its loop.
template <class T, class TL>
__device__ __forceinline__ void store_output(const Params& p, const WaveState<TL>& ws,
                                             lds_t* smem, long long o_off, long long lse_off,
                                             int qt, int qw, int lane) {
  constexpr int QB = TL::QB, DB = TL::D / 32;
  const int lr = lane & 31;
  const int hh = lane >> 5;
  const bool staged = TL::STAGE_O && !p.o_f32;
  lds_t* const stage = smem + TL::STAGE_OFF + qw * QB * 32 * TL::SROW;
  // Columns db·32 + 16·hh + [0, 8) and [8, 16) of the lane's row, rounded.
  auto pack16 = [&](int qb, int db, float inv, u32x4_t& w0, u32x4_t& w1) {
    uint32_t w[8];
#pragma unroll
    for (int i = 0; i < 8; ++i)
      w[i] = Mma<T>::pack(ws.o[qb][db][2 * i] * inv, ws.o[qb][db][2 * i + 1] * inv);
    w0 = u32x4_t{w[0], w[1], w[2], w[3]};
    w1 = u32x4_t{w[4], w[5], w[6], w[7]};
  };
#pragma unroll
  for (int qb = 0; qb < QB; ++qb) {
    const float lt = lane_pair_sum(ws.l[qb]);
    const int row = qt * TL::BM + (qw * QB + qb) * 32 + lr;
    // lt == 0 only for a row without any valid key (causal): O = 0, LSE = -inf.
    const float inv = lt > 0.f ? 1.0f / lt : 0.f;
    if (staged) {
      lds_t* srow = stage + (qb * 32 + lr) * TL::SROW;
#pragma unroll
      for (int db = 0; db < DB; ++db) {
        u32x4_t w0, w1;
        pack16(qb, db, inv, w0, w1);
        st_lds16(srow + db * 64 + 32 * hh, w0);
        st_lds16(srow + db * 64 + 32 * hh + 16, w1);
      }
    }
    if (row < p.Sq) {
      const long long ro = o_off + (long long)row * p.o_ss;
      if (p.o_f32) {
        float* orow = static_cast<float*>(p.o) + ro;
#pragma unroll
        for (int db = 0; db < DB; ++db)
#pragma unroll
          for (int j = 0; j < 4; ++j) {
            u32x4_t w;
#pragma unroll
            for (int e = 0; e < 4; ++e) w[e] = f2u(ws.o[qb][db][4 * j + e] * inv);
            *reinterpret_cast<u32x4_t*>(orow + db * 32 + 16 * hh + 4 * j) = w;
          }
      } else if (!staged) {
        uint16_t* orow = static_cast<uint16_t*>(p.o) + ro;
#pragma unroll
        for (int db = 0; db < DB; ++db) {
          u32x4_t w0, w1;
          pack16(qb, db, inv, w0, w1);
          *reinterpret_cast<u32x4_t*>(orow + db * 32 + 16 * hh) = w0;
          *reinterpret_cast<u32x4_t*>(orow + db * 32 + 16 * hh + 8) = w1;
        }
      }
      if (p.lse != nullptr && hh == 0) {
        // ln(sum_j exp(s_j * scale)) = (m + log2(l)) * ln 2
        p.lse[lse_off + row] = lt > 0.f ? (ws.m[qb] + __builtin_amdgcn_logf(lt)) * 0.69314718055994531f
                                        : -__builtin_inff();
      }
    }
  }
  if (staged) {
    // Read back as whole rows: 16-byte chunk i·64 + lane of the wave's rows.
    constexpr int CPR = TL::D / 8;
    constexpr int NRD = QB * 32 * CPR / 64;
    static_assert(QB * 32 * CPR % 64 == 0, "staged rows fill whole instructions");
    const int row0 = qt * TL::BM + qw * QB * 32;
    uint16_t* const ob = static_cast<uint16_t*>(p.o) + o_off;
    u32x4_t x[NRD];
#pragma unroll
    for (int i = 0; i < NRD; ++i) {
      const int ch = i * 64 + lane;
      x[i] = ld_lds16(stage + (ch / CPR) * TL::SROW + (ch % CPR) * 16);
    }
#pragma unroll
    for (int i = 0; i < NRD; ++i) {
      const int ch = i * 64 + lane;
      const int r = row0 + ch / CPR;
      if (r < p.Sq) *reinterpret_cast<u32x4_t*>(ob + (long long)r * p.o_ss + (ch % CPR) * 8) = x[i];
    }
  }
}


// ---- ping-pong schedule ------------------------------------------------------
//
// Every wave runs the same sequence of phases, separated by workgroup
// barriers:  M(i) = Sᵀ of tile i then P·V of tile i-1 (MFMA, with the first
// half of tile i's softmax between the P·V MFMAs),  V(i) = the rest of the
// softmax of tile i (VALU).  With 8 waves, waves w and w+4 share a SIMD; group 1
// (waves 4-7) starts one barrier later than group 0, so on every SIMD one wave
// keeps the MFMA unit busy while the other keeps the VALU busy:
//     slot 2i:   group 0 M(i)     group 1 V(i-1)
//     slot 2i+1: group 0 V(i)     group 1 M(i)
// (the producer/consumer overlap that the warp-specialised kernels of "B200
// Attention Kernel from Scratch to Near-SOTA in 60 Diagrams", Chapter 4 - Warp
// Specialization, and "Attention for sm90, Line by Line", "Why does a flash
// attention kernel need three warpgroups?", obtain with separate roles).
// K/V copies are issued and awaited only in VALU phases (and, for group 1, at
// the end of an MFMA phase), so the MFMA phase issues nothing but MFMAs and
// their LDS operand reads; the three-deep ring makes that legal (see
// process_item).

// ---- split softmax: its first half rides in the MFMA phase --------------------
//
// M(i) issues the Sᵀ MFMAs of tile i first and the P·V MFMAs of tile i-1
// after them.  Once Sᵀ is complete, the first half of the
// softmax of tile i runs between the P·V MFMAs, in issue slots the MFMA phase
// leaves idle: the row maximum, the threshold-guarded move of m, and
// s·c - m (in place).  V(i) is left with exp2, the row sums, the packing of P
// and the rescale of O.  The work is laid out as slots of one MFMA each;
// operands are read from LDS two slots ahead, and scheduling barriers keep
// every slot's work in place.

// LDS operands of an MFMA phase.  Slot s reads a K fragment for an Sᵀ MFMA
// (key block s % NB, head-dim step s / NB) or a V fragment for a P·V MFMA:
// lane group g = lane/16 covers key half g/2 and head-dim half g%2; inside
// the group, lane i reads key row i/4 and the 8-byte piece of head-dim
// columns chosen so that the transposed result is lane_key-ordered.  Slot
// order: all Sᵀ slots then all P·V slots, or with ALT (and both kinds
// present) Sᵀ in the even slots and P·V in the odd ones.
template <class TL, bool QK, bool PV>
struct Operands {
  static constexpr int NB = TL::BN / 32, DT = TL::D / 16, DB = TL::D / 32;
  static constexpr int NQ = QK ? NB * DT : 0;       // Sᵀ MFMAs
  static constexpr int NP = PV ? NB * 2 * DB : 0;   // P·V MFMAs
  static constexpr int NS = NQ + NP;
  static constexpr bool IL = TL::ALT && QK && PV && NQ == NP;
  static constexpr bool is_qk(int s) { return IL ? s % 2 == 0 : s < NQ; }
  static constexpr int qk_index(int s) { return IL ? s / 2 : s; }
  static constexpr int pv_index(int s) { return IL ? s / 2 : s - NQ; }
  const lds_t* kbase;
  const lds_t* vbase;
  const lds_t* vbase1;

  __device__ __forceinline__ Operands(const lds_t* kl, const lds_t* vl, int lane) {
    const int g = lane >> 4;
    const int li = lane & 15;
    uint32_t ka = (uint32_t)(uintptr_t)kl + (uint32_t)((lane & 31) * TL::KS + (lane >> 5) * 16);
    const int vrow = 16 * (g >> 1) + (li >> 2);
    int vchunk = 2 * (li & 1) + (g & 1);
    if (TL::VSWZ) vchunk ^= ((vrow >> 1) & 1) << 2;
    uint32_t va = (uint32_t)(uintptr_t)vl + (uint32_t)(vrow * TL::VS + vchunk * 16 + ((li >> 1) & 1) * 8);
    // Swizzled V: the second 64 bytes of a row (db = 1) sit at the address
    // with bit 6 flipped, which no immediate offset expresses; a second base.
    uint32_t va1 = va ^ 64u;
    if (QK) asm volatile("" : "+v"(ka));
    if (PV) asm volatile("" : "+v"(va));
    if (PV && TL::VSWZ) asm volatile("" : "+v"(va1));
    kbase = (const lds_t*)(uintptr_t)ka;
    vbase = (const lds_t*)(uintptr_t)va;
    vbase1 = (const lds_t*)(uintptr_t)va1;
  }

  __device__ __forceinline__ u32x4_t frag(int s) const {
    if (is_qk(s)) {
      const int q = qk_index(s);
      return ld_lds16(kbase + (q % NB) * 32 * TL::KS + (q / NB) * 32);
    }
    const int i = pv_index(s);
    const int nb = i / (2 * DB), mm = (i / DB) % 2, db = i % DB;
    const lds_t* pv0 = (TL::VSWZ ? (db == 0 ? vbase : vbase1) : vbase + db * 64) +
                       (nb * 32 + 8 * mm) * TL::VS;
    const u32x2_t lo = ld_lds_tr(pv0);
    const u32x2_t hi = ld_lds_tr(pv0 + 4 * TL::VS);
    const u32x4_t a = {lo[0], lo[1], hi[0], hi[1]};
    return a;
  }
};

// STEADY: a step of the steady loop, where every row's kept maximum is already
// finite (tile 0 of the item, or of the group, was visible to every row), so
// the guards for m = -inf are left out.
template <class T, class TL, bool QK, bool PV, bool STEADY = false>
__device__ __forceinline__ void mma_phase(WaveState<TL>& ws, const lds_t* kl, const lds_t* vl,
                                          SAcc<TL>& sacc, const PFrag<TL>& pfr,
                                          float (&mprev)[TL::QB], float (&mu)[TL::QB], float c,
                                          int lane) {
  using Op = Operands<TL, QK, PV>;
  constexpr int QB = TL::QB, NB = Op::NB, DB = Op::DB;
  constexpr int NQ = Op::NQ, NP = Op::NP, NS = Op::NS;
  constexpr int NV = NB * 16;            // scores per lane per 32-query block
  static_assert(NS >= 1, "empty phase");
  constexpr bool IL = Op::IL;
  const Op op(kl, vl, lane);
  constexpr int LD = 2;  // operands are read two slots ahead
  if (TL::PRIO) __builtin_amdgcn_s_setprio(3);
  u32x4_t fr[NS];
#pragma unroll
  for (int j = 0; j < LD && j < NS; ++j) fr[j] = op.frag(j);

  // First half of the softmax of the new Sᵀ: x = s·c - mu in place, one unit
  // per score.  mu is the kept maximum m (0 while m is still -inf, so that no
  // (-inf) - (-inf) is formed); mprev keeps m for softmax_tail, which decides
  // whether the maximum moves.
  float nm[QB];
  if (QK) {
#pragma unroll
    for (int qb = 0; qb < QB; ++qb) {
      const float mold = ws.m[qb];
      mprev[qb] = mold;
      mu[qb] = (!STEADY && mold == -__builtin_inff()) ? 0.f : mold;
      nm[qb] = -mu[qb];
    }
  }
  constexpr int NU = QK ? QB * NV : 0;
  auto unit = [&](int k) {
    const int qb = k / NV, v = k % NV;
    float y = __builtin_fmaf(sacc[qb][v / 16][v % 16], c, nm[qb]);
    asm volatile("" : "+v"(y));  // keep it here, not sunk into the VALU phase
    sacc[qb][v / 16][v % 16] = y;
  };
  // Units ride on the P·V slots from the third on, when the Sᵀ results have
  // landed; without P·V (the first tile), or with alternating slots, they run
  // after the last MFMA.
  constexpr int FIRST = NQ + 2;
  constexpr int SLOTS = NS - FIRST;
  const f32x16_t zero = {};
#pragma unroll
  for (int s = 0; s < NS; ++s) {
    if (Op::is_qk(s)) {
      const int q = Op::qk_index(s);
      const int nb = q % NB, t = q / NB;
#pragma unroll
      for (int qb = 0; qb < QB; ++qb)
        sacc[qb][nb] = Mma<T>::mfma(fr[s], ws.qf[qb][t], t == 0 ? zero : sacc[qb][nb]);
    } else {
      const int i = Op::pv_index(s);
      const int nb = i / (2 * DB), mm = (i / DB) % 2, db = i % DB;
#pragma unroll
      for (int qb = 0; qb < QB; ++qb) {
        const u32x4_t b = {pfr[qb][nb][4 * mm + 0], pfr[qb][nb][4 * mm + 1],
                           pfr[qb][nb][4 * mm + 2], pfr[qb][nb][4 * mm + 3]};
        ws.o[qb][db] = Mma<T>::mfma(fr[s], b, ws.o[qb][db]);
      }
    }
    if (s + LD < NS) fr[s + LD] = op.frag(s + LD);
    if (!IL && SLOTS > 0 && s >= FIRST) {
      // Slot FIRST + j takes units u with floor(u·SLOTS/NU) == j.
      const int j = s - FIRST;
      const int u0 = (j * NU + SLOTS - 1) / SLOTS, u1 = ((j + 1) * NU + SLOTS - 1) / SLOTS;
#pragma unroll
      for (int u = u0; u < u1; ++u) unit(u);
    }
    __builtin_amdgcn_sched_barrier(0);
  }
  if (IL || SLOTS <= 0) {
#pragma unroll
    for (int u = 0; u < NU; ++u) unit(u);
  }
  if (TL::PRIO) __builtin_amdgcn_s_setprio(0);
}

// Second half of the softmax of tile i; sacc holds x = s·c - mu.
//
// The lazy rescale (reading of "B200 Attention Kernel from Scratch to
// Near-SOTA in 60 Diagrams", Chapter 11) moves the kept maximum m only when a
// tile's row maximum exceeds it by more than thr.  Instead of taking every
// tile's maximum, p = 2^x is computed against the kept m first, and its
// lane-partial row sum in fp32 (for fp16, the sum of P rounded to fp16; see
// Mma<F16>::sum2).  A lane whose partial row sum is at most 2^thr has every
// p <= 2^thr, so none of its scores exceeds m + thr (up to P's rounding) and
// its row keeps m.  Masked keys get x = -inf first, so their p is 0 and the
// same test holds on masked tiles.  Only when some lane of the wave fails
// that test (or m is still -inf) does the wave take the maxima: each row's
// maximum over its visible keys, max(x) + mu, against m, the
// threshold-guarded move, the shift to the new reference, and P and its sums
// again.  Rows that keep m get the same P either way.  Then l = l·alpha + ΣP
// and, if a row of the wave moved its maximum, O·alpha.  Issued as wide
// independent passes.
template <class T, class TL, bool MASK, bool GUARD, bool STEADY = false>
__device__ __forceinline__ void softmax_tail(WaveState<TL>& ws, float (&alpha)[TL::QB], bool& any,
                                             SAcc<TL>& sacc, PFrag<TL>& pfr,
                                             const float (&mprev)[TL::QB],
                                             const float (&mu)[TL::QB], int kb, int klim,
                                             float thr, float psum_max, int lane) {
  constexpr int QB = TL::QB, NV = TL::BN / 32 * 16;
  int lim = klim - (kb + 16 * (lane >> 5));
  if (MASK) {
    asm volatile("" : "+v"(lim));
#pragma unroll
    for (int qb = 0; qb < QB; ++qb)
#pragma unroll
      for (int v = 0; v < NV; ++v)
        if ((v / 16) * 32 + (v % 16) >= lim) sacc[qb][v / 16][v % 16] = -__builtin_inff();
  }
  auto exp2_all = [&](float (&e)[QB][NV], const float (&sh)[QB]) {
#pragma unroll
    for (int qb = 0; qb < QB; ++qb)
#pragma unroll
      for (int v = 0; v < NV; ++v) {
        const float x = sacc[qb][v / 16][v % 16] - sh[qb];
        e[qb][v] = (TL::POLY > 0 && v % (TL::POLY > 0 ? TL::POLY : 1) == 0) ? exp2_poly(x)
                                                                             : __builtin_amdgcn_exp2f(x);
      }
  };
  // Lane-partial row sums.  fp16: P rounded and packed (the B operand of the
  // next P·V) first, then the sums of exactly that P, one dot2 per packed
  // pair.  bf16: the sums of the fp32 p; P is packed after the last pass.
  auto pack_sums = [&](float (&e)[QB][NV], float (&ls)[QB]) {
#pragma unroll
    for (int qb = 0; qb < QB; ++qb) {
      // v_exp_f32 gives exactly 0 for the masked keys' -inf; exp2_poly clamps
      // its argument, so its masked p are cleared here.
      if (MASK && TL::POLY > 0) {
#pragma unroll
        for (int v = 0; v < NV; ++v)
          if ((v / 16) * 32 + (v % 16) >= lim) e[qb][v] = 0.f;
      }
      float l4[4];
      if (Mma<T>::PACKED_SUMS) {
#pragma unroll
        for (int w = 0; w < NV / 2; ++w)
          pfr[qb][w / 8][w % 8] = Mma<T>::pack(e[qb][2 * w], e[qb][2 * w + 1]);
#pragma unroll
        for (int w = 0; w < 4; ++w) l4[w] = Mma<T>::sum2(pfr[qb][w / 8][w % 8], 0.f);
#pragma unroll
        for (int w = 4; w < NV / 2; ++w) l4[w & 3] = Mma<T>::sum2(pfr[qb][w / 8][w % 8], l4[w & 3]);
      } else {
#pragma unroll
        for (int v = 0; v < 4; ++v) l4[v] = e[qb][v];
#pragma unroll
        for (int v = 4; v < NV; ++v) l4[v & 3] += e[qb][v];
      }
      ls[qb] = (l4[0] + l4[1]) + (l4[2] + l4[3]);
    }
  };
  float e[QB][NV], ls[QB], sh[QB];
#pragma unroll
  for (int qb = 0; qb < QB; ++qb) {
    sh[qb] = 0.f;
    alpha[qb] = 1.f;
  }
  any = false;
  // One pass in the common case.  A second pass, after the maxima moved the
  // reference, recomputes P and its sums with the same code (a single
  // definition of P keeps register use as in one pass).
  bool again = false;
#pragma nounroll
  for (;;) {
    exp2_all(e, sh);
    __builtin_amdgcn_sched_barrier(0);
    pack_sums(e, ls);
    if (again) break;
    bool need = false;
#pragma unroll
    for (int qb = 0; qb < QB; ++qb)
      need = need || (!STEADY && mprev[qb] == -__builtin_inff()) || !(ls[qb] <= psum_max);
    if (__builtin_amdgcn_ballot_w64(need) == 0) break;
#pragma unroll
    for (int qb = 0; qb < QB; ++qb) {
      float m4[4] = {-__builtin_inff(), -__builtin_inff(), -__builtin_inff(), -__builtin_inff()};
#pragma unroll
      for (int v = 0; v < NV; ++v) m4[v & 3] = fmaxf(m4[v & 3], sacc[qb][v / 16][v % 16]);
      const float tx = lane_pair_max(fmaxf(fmaxf(m4[0], m4[1]), fmaxf(m4[2], m4[3])));
      const float mcand = tx + mu[qb];  // tile row maximum over visible keys, log2 units
      const float mold = mprev[qb];
      const bool rebase = (mold == -__builtin_inff()) || (mcand > mold + thr);
      const float mnew = rebase ? mcand : mold;
      const float mref = (GUARD && mnew == -__builtin_inff()) ? 0.f : mnew;
      alpha[qb] = __builtin_amdgcn_exp2f(mold - mref);  // 1 if kept, 0 on the first tile
      any = any || (__builtin_amdgcn_ballot_w64(rebase) != 0);
      ws.m[qb] = mnew;
      sh[qb] = mref - mu[qb];
    }
    again = true;
  }
#pragma unroll
  for (int qb = 0; qb < QB; ++qb) {
    ws.l[qb] = ws.l[qb] * alpha[qb] + ls[qb];
    if (!Mma<T>::PACKED_SUMS) {
#pragma unroll
      for (int w = 0; w < NV / 2; ++w)
        pfr[qb][w / 8][w % 8] = Mma<T>::pack(e[qb][2 * w], e[qb][2 * w + 1]);
    }
  }
  // O has received P·V of tile i-1 and not yet that of tile i.
  if (any) rescale_o(ws, alpha);
}

// Key-split merge: group 1 hands its (m, l, O) to the wave of group 0 that
// holds the same query rows, through LDS (the rings are idle at this point),
// and group 0 combines the two partial results of each row:
//   m = max(m0, m1),  l = l0·2^(m0-m) + l1·2^(m1-m),  O = O0·2^(m0-m) + O1·2^(m1-m).
// (The associative merge of partial softmax results: "Attention for sm90, Line
// by Line", the split-KV discussion, and the running-max algebra of "B200
// Attention Kernel from Scratch to Near-SOTA in 60 Diagrams", Chapter 1.)
template <class TL>
__device__ __forceinline__ void merge_key_halves(WaveState<TL>& ws, lds_t* smem, int grp, int qw,
                                                 int lane) {
  constexpr int QB = TL::QB, DB = TL::D / 32;
  lds_t* xb = smem + (qw * TL::XCH * 64 + lane) * 16;
  auto slot = [&](int c) { return xb + c * 1024; };
  if (grp == 1) {
#pragma unroll
    for (int qb = 0; qb < QB; ++qb)
#pragma unroll
      for (int db = 0; db < DB; ++db)
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          const u32x4_t w = {f2u(ws.o[qb][db][4 * j]), f2u(ws.o[qb][db][4 * j + 1]),
                             f2u(ws.o[qb][db][4 * j + 2]), f2u(ws.o[qb][db][4 * j + 3])};
          st_lds16(slot((qb * DB + db) * 4 + j), w);
        }
    static_assert(QB <= 2, "(m, l) of every query block share one chunk");
    u32x4_t ml = {0u, 0u, 0u, 0u};
#pragma unroll
    for (int qb = 0; qb < QB; ++qb) {
      ml[2 * qb] = f2u(ws.m[qb]);
      ml[2 * qb + 1] = f2u(ws.l[qb]);
    }
    st_lds16(slot(TL::XCH - 1), ml);
  }
  __syncthreads();
  if (grp == 0) {
    const u32x4_t ml = ld_lds16(slot(TL::XCH - 1));
#pragma unroll
    for (int qb = 0; qb < QB; ++qb) {
      const float m1 = u2f(ml[2 * qb]);
      const float l1 = u2f(ml[2 * qb + 1]);
      const float m0 = ws.m[qb];
      const float mm = fmaxf(m0, m1);
      // A row without a visible key in either half keeps m = -inf and l = 0.
      const bool none = mm == -__builtin_inff();
      const float a0 = none ? 0.f : __builtin_amdgcn_exp2f(m0 - mm);
      const float a1 = none ? 0.f : __builtin_amdgcn_exp2f(m1 - mm);
      ws.m[qb] = mm;
      ws.l[qb] = ws.l[qb] * a0 + l1 * a1;
#pragma unroll
      for (int db = 0; db < DB; ++db)
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          const u32x4_t w = ld_lds16(slot((qb * DB + db) * 4 + j));
#pragma unroll
          for (int e = 0; e < 4; ++e)
            ws.o[qb][db][4 * j + e] =
                __builtin_fmaf(ws.o[qb][db][4 * j + e], a0, u2f(w[e]) * a1);
        }
    }
  }
  // The exchange area is ring memory again for the next item's copies.
  __syncthreads();
}

// Geometry of one work item as one wave sees it: item -> (KV range sp, head
// bh, query tile qt), the keys the item sees, and this wave group's share.
struct ItemGeom {
  int qt, bh, sp, b, h, k0, S, nt, t_mask, klim, nt0, tb, ntg, Sg, klg;
  bool ragged;
  const uint16_t* qh;
  const uint16_t* kh;
  const uint16_t* vh;
};

template <class TL, bool CAUSAL>
__device__ __forceinline__ ItemGeom item_geom(const Params& p, int item, int grp, int qw, int lr) {
  constexpr int BN = TL::BN;
  constexpr bool KSPLIT = TL::KSPLIT;
  ItemGeom g;
  // Non-causal: consecutive items are the query tiles of one head and one KV
  // range.  Causal: the last (longest) query tiles of every head come first,
  // so that workgroups dispatched in order start with the largest items;
  // consecutive items are different heads, and head bh lands on XCD bh % 8
  // when B·H % 8 == 0.
  int t_;
  if (CAUSAL) {
    g.bh = item % p.BH;
    t_ = item / p.BH;
    g.qt = p.n_qtiles - 1 - t_ % p.n_qtiles;
    g.sp = t_ / p.n_qtiles;
  } else {
    g.qt = item % p.n_qtiles;
    t_ = item / p.n_qtiles;
    g.bh = t_ % p.BH;
    g.sp = t_ / p.BH;
  }
  g.b = g.bh / p.H;
  g.h = g.bh - g.b * p.H;
  g.k0 = g.sp * p.split_len;
  // S (keys of this item's range) passes through an empty asm so that per-lane
  // values derived from it (tail masks, clamped copy addresses) are recomputed
  // per item instead of being hoisted out of the persistent loop, where they
  // would occupy registers for the whole kernel.
  int S = min(p.Skv - g.k0, p.split_len);
  asm volatile("" : "+s"(S));
  g.S = S;
  g.qh = p.q + g.b * p.q_sb + g.h * p.q_sh;
  // Keys of the range visible to this item: all S, or with a causal mask the
  // prefix that its last query row sees.  Whole tiles below t_mask are
  // visible to every row of the item and carry no mask.
  g.klim = S;  // this lane's key limit, counted from the range start
  if (CAUSAL) {
    const int q_first = g.qt * TL::BM;
    const int q_last = min(p.Sq, q_first + TL::BM) - 1;
    const int seen = min(S, q_last + p.coff - g.k0 + 1);
    g.nt = seen > 0 ? (seen + BN - 1) / BN : 0;
    g.t_mask = min(max(q_first + p.coff - g.k0 + 1, 0), S) / BN;
    const int row = q_first + qw * 32 + lr;
    g.klim = min(S, max(row + p.coff - g.k0 + 1, 0));
  } else {
    g.nt = (S + BN - 1) / BN;
    g.t_mask = S / BN;
  }
  g.ragged = (S % BN) != 0;
  // This group's tiles: all nt, or with a key split the first ceil(nt/2)
  // (group 0) or the rest (group 1, starting at tile tb).  Sg and klg count
  // keys from the group's first tile.
  g.nt0 = KSPLIT ? (g.nt + 1) / 2 : g.nt;
  g.tb = (KSPLIT && grp == 1) ? g.nt0 : 0;
  g.ntg = (KSPLIT && grp == 1) ? g.nt - g.nt0 : g.nt0;
  g.Sg = S - g.tb * BN;
  g.klg = g.klim - g.tb * BN;
  g.kh = p.k + g.b * p.k_sb + g.h * p.k_sh + (long long)(g.k0 + g.tb * BN) * p.k_ss;
  g.vh = p.v + g.b * p.v_sb + g.h * p.v_sh + (long long)(g.k0 + g.tb * BN) * p.v_ss;
  return g;
}

// Copy set c(t) = {K_t, V_{t-1}} of an item: the tiles M(t) reads.  Each wave
// issues its share; tiles that run past the group's last key are clamped.
template <class TL>
__device__ __forceinline__ void issue_copy_set(const Params& p, const Copies<TL>& cp,
                                               const ItemGeom& g, const Ring<TL>& ring, int t,
                                               int qw, int lane) {
  constexpr int BN = TL::BN;
  if (t < g.ntg) {
    const uint16_t* kt = g.kh + (long long)(t * BN) * p.k_ss;
    if ((t + 1) * BN <= g.Sg)
      cp.k.issue(kt, ring.k(t), qw);
    else
      cp.k.issue_clamped(kt, g.Sg - t * BN, (uint32_t)p.k_ss * 2u, ring.k(t), qw, lane);
  }
  if (t >= 1 && t <= g.ntg) {
    const int u = t - 1;
    const uint16_t* vt = g.vh + (long long)(u * BN) * p.v_ss;
    if ((u + 1) * BN <= g.Sg)
      cp.v.issue(vt, ring.v(u), qw);
    else
      cp.v.issue_clamped(vt, g.Sg - u * BN, (uint32_t)p.v_ss * 2u, ring.v(u), qw, lane);
  }
}

// Prologue of an item: c(0) (and with copies two tiles ahead, on three-deep
// rings and on every key-split ring, c(1)) and the wave's Q rows into the
// MFMA B-operand registers.  Rows past Sq load row Sq-1 instead: they are
// computed on that copy and never stored, and the loads need no lane mask
// (a masked load into zeroed registers made the compiler wait for every
// vector memory operation in flight, the copies just issued included).
template <class TL>
__device__ __forceinline__ void item_prologue(const Params& p, const Copies<TL>& cp,
                                              const ItemGeom& g, const Ring<TL>& ring,
                                              WaveState<TL>& ws, int qw, int lane) {
  constexpr bool DEEP = TL::STAGES == 3 || TL::KSPLIT;
  constexpr int QB = TL::QB, DT = TL::D / 16;
  if (g.ntg > 0) {
    issue_copy_set<TL>(p, cp, g, ring, 0, qw, lane);
    if (DEEP) issue_copy_set<TL>(p, cp, g, ring, 1, qw, lane);
  }
  const int lr = lane & 31;
  const int hh = lane >> 5;
#pragma unroll
  for (int qb = 0; qb < QB; ++qb) {
    const int row = min(g.qt * TL::BM + (qw * QB + qb) * 32 + lr, p.Sq - 1);
#pragma unroll
    for (int t = 0; t < DT; ++t) ws.qf[qb][t] = ld_global16(g.qh + (long long)row * p.q_ss + 16 * t + 8 * hh);
  }
}

// One work item.  `pre` < 0: the item's prologue is issued here; otherwise the
// previous item already issued it ahead of its own O stores, and `pre` is the
// number of those stores that may still be in flight when the prologue's
// copies and Q rows have landed (vector memory operations complete in issue
// order).  With a next item (non-causal persistent grids), this item issues
// the next one's prologue once its own K/V reads are over, ahead of its
// stores, and returns the `pre` for it; otherwise it returns -1.  All work
// items reach their ends at about the same time, so their O stores form one
// burst of HBM writes: the next item's copies and Q rows no longer queue
// behind it, and the stores drain during the next item's first slots.
template <class T, class TL, bool CAUSAL>
__device__ __forceinline__ int process_item(const Params& p, const Copies<TL>& cp, lds_t* smem,
                                            int item, int next, int wave, int lane,
                                            WaveState<TL>& ws, int pre) {
  constexpr int D = TL::D, BN = TL::BN, QB = TL::QB, DB = D / 32;
  constexpr bool KSPLIT = TL::KSPLIT;
  // O store instructions of a wave whose rows are all below Sq, direct or
  // staged through LDS (at least; more with fp32 partials or the LSE).
  constexpr int NST = QB * DB * 2;
  static_assert(!CAUSAL || QB == 1, "causal masks assume one 32-query block per wave");
  const int lr = lane & 31;
  // Wave groups: waves w and w+4 share a SIMD.  grp decides the slot offset
  // of the ping-pong schedule.  Without a key split the groups hold different
  // query rows and consume one K/V stream, whose copies they share; group 1
  // trails by one slot.  With a key split both groups hold the same query rows
  // (qw) and each streams its own keys, so each runs the leading group's copy
  // schedule on its own ring (`lead`).
  const int grp = TL::NW == 8 ? (wave >> 2) : 0;
  const int qw = KSPLIT ? (wave & 3) : wave;
  const bool lead = KSPLIT || grp == 0;
  const ItemGeom g = item_geom<TL, CAUSAL>(p, item, grp, qw, lr);
  const int qt = g.qt, bh = g.bh, sp = g.sp, b = g.b, h = g.h;
  const int nt = g.nt, t_mask = g.t_mask;
  const bool ragged = g.ragged;
  const float c = p.c, thr = p.thr;
  // A lane's partial row sum of p = 2^(s·c - m) up to this bound proves that
  // none of its scores exceeds m + thr (see softmax_tail).
  const float psum_max = __builtin_amdgcn_exp2f(thr);
  const int kss = p.k_ss, vss = p.v_ss;

  if (CAUSAL && nt == 0) {
    // No query row of this item sees a key of the range: O = 0, LSE = -inf.
    if (KSPLIT && grp == 1) return -1;
    WaveState<TL> wz;
#pragma unroll
    for (int qb = 0; qb < QB; ++qb) {
      wz.m[qb] = -__builtin_inff();
      wz.l[qb] = 0.f;
#pragma unroll
      for (int db = 0; db < DB; ++db)
#pragma unroll
        for (int i = 0; i < 16; ++i) wz.o[qb][db][i] = 0.f;
    }
    store_output<T, TL>(p, wz, smem, sp * p.o_split + b * p.o_sb + h * p.o_sh,
                       sp * p.lse_split + (long long)bh * p.Sq, qt, qw, lane);
    return -1;
  }

  const int nt0 = g.nt0, tb = g.tb, ntg = g.ntg, klg = g.klg;
  const uint16_t* __restrict__ kh = g.kh;
  const uint16_t* __restrict__ vh = g.vh;
  const Ring<TL> ring{smem + (KSPLIT ? grp * TL::RING_BYTES : 0)};
  auto copy_set = [&](int t) { issue_copy_set<TL>(p, cp, g, ring, t, qw, lane); };
  constexpr bool DEEP = TL::STAGES == 3 || TL::KSPLIT;
  if (pre < 0) item_prologue<TL>(p, cp, g, ring, ws, qw, lane);
#pragma unroll
  for (int qb = 0; qb < QB; ++qb) {
    ws.m[qb] = -__builtin_inff();
    ws.l[qb] = 0.f;
#pragma unroll
    for (int db = 0; db < DB; ++db)
#pragma unroll
      for (int i = 0; i < 16; ++i) ws.o[qb][db][i] = 0.f;
  }
  if (pre > 0) wait_vmem_n<NST>();
  else wait_vmem();
  __syncthreads();

  // Slots: group 0 runs M(i) in slot 2i and V(i) in slot 2i+1, group 1 one
  // slot later.  Copies are issued only in V phases: in V(i) a wave issues its
  // share of c(i + ahead).  A wave's share of c(i+1) is complete before the
  // barrier that ends the slot before M(i+1): the leading schedule waits in
  // V(i); group 1 of a shared stream waits at the end of M(i).
  //  * three-deep ring: ahead = 2; the leading schedule waits at the start of
  //    V(i).  c(i+2) overwrites K_{i-1} and V_{i-2}, last read in M(i-1),
  //    two slots or more before V(i).
  //  * two-deep ring of one group (key split): as three-deep.  c(i+2) issued
  //    in V(i) overwrites K_i and V_{i-1}, which only this group's M(i)
  //    reads, and M(i) ends before V(i).
  //  * two-deep shared ring: ahead = 1 for the leading schedule, which waits
  //    at the end of V(i) (after its softmax), and 2 for group 1.  c(i+1)
  //    issued in V(i) overwrites K_{i-1} and V_{i-2} (read in M(i-1), which
  //    ends before V(i) of either group starts); c(i+2) issued by group 1 in
  //    slot 2i+2 overwrites K_i and V_{i-1}, read in slots 2i and 2i+1.
  //  * three-deep shared ring, group 1 (G1A3): ahead = 3.  Its V(i) falls in
  //    slot 2i+2, and c(i+3) overwrites K_i and V_{i-1}, read in M(i) of both
  //    groups (slots 2i and 2i+1).  At the end of its M(i) (slot 2i+1) it
  //    needs its share of c(i+1), issued in slot 2i-2; in the steady loop it
  //    waits only for that, letting the share of c(i+2) issued since stay in
  //    flight (with ahead = 2 the share of c(i+1) would have been issued one
  //    slot before, and the wait showed at that barrier).
  // No DMA is issued or awaited inside a leading MFMA phase.
  constexpr bool G1A3 = TL::STAGES == 3 && !TL::KSPLIT && TL::NW == 8;
  const int ahead = (!lead && G1A3) ? 3 : (DEEP || !lead) ? 2 : 1;
  SAcc<TL> sacc;
  PFrag<TL> pfr;
  if (grp == 1) {  // group 1 sits out slot 0
    if (!lead && !DEEP) copy_set(1);
    if (!lead && G1A3) copy_set(2);
    __syncthreads();
  }
  // Softmax state handed from M(i) to V(i): rescale factors, the maximum
  // before tile i and the reference the scores were shifted by.
  float alpha[QB], mprev[QB], mu[QB];
  bool any = false;
  // M(i): Sᵀ of tile i (unless i == ntg) and P·V of tile i-1 (unless i == 0),
  // with the first half of tile i's softmax; V(i): the rest of the softmax of
  // tile i, masked (MK) when it is not a whole tile visible to every row.
#define ATTN_MPHASE(I, QK, PV)                                                                     \
  mma_phase<T, TL, QK, PV>(ws, QK ? ring.k(I) : nullptr, PV ? ring.v((I) - 1) : nullptr, sacc, pfr, \
                           mprev, mu, c, lane)
#define ATTN_VPHASE(I, MK)                                                                         \
  softmax_tail<T, TL, MK, CAUSAL>(ws, alpha, any, sacc, pfr, mprev, mu, (I) * BN, klg, thr,        \
                                  psum_max, lane)
  if (ntg > 0) {
    // One step i: M(i), then V(i).  `cset` issues the step's copies.
    auto step = [&](int i, auto cset, bool masked) {
      if (i == 0) ATTN_MPHASE(0, true, false);
      else ATTN_MPHASE(i, true, true);
      if (!lead) wait_vmem();
      __syncthreads();
      if (DEEP && lead) wait_vmem();
      cset();
      if (masked) ATTN_VPHASE(i, true);
      else ATTN_VPHASE(i, false);
      if (!DEEP && lead) wait_vmem();
      __syncthreads();
    };
    auto masked = [&](int i) { return tb + i >= t_mask || (tb + i == nt - 1 && ragged); };
    step(0, [&]() { copy_set(ahead); }, masked(0));
    // Steps 1 .. steady copy only whole tiles and softmax unmasked tiles; the
    // remaining (at least the last three) steps are peeled so the steady loop
    // carries no such branches.  A schedule that copies three tiles ahead
    // stops one step earlier: its step ntg-4 copies the last, maybe ragged,
    // tile.  (Every step passes the same two barriers, steady or peeled.)
    const int steady = (CAUSAL ? min(ntg - 4, t_mask - tb - 1) : ntg - 4) - (ahead == 3 ? 1 : 0);
    // Steady step i.  With copies two tiles ahead the loop is unrolled by the
    // ring depth, so every ring buffer a step touches (K_i, V_{i-1}, and the
    // copy targets K_{i+2}, V_{i+1}) is a compile-time offset: RR carries
    // i % STAGES, or -1 where it is computed at run time.  This takes the
    // modulo arithmetic and most address set-up out of the VALU phase.
    auto steady_step = [&](int i, auto RR) {
      constexpr int R = decltype(RR)::value;
      constexpr int NS = TL::STAGES;
      lds_t* const vbase = ring.base + NS * TL::K_TILE;
      lds_t* const k_i = R >= 0 ? ring.base + R * TL::K_TILE : ring.k(i);
      lds_t* const v_im1 = R >= 0 ? vbase + ((R + NS - 1) % NS) * TL::V_TILE : ring.v(i - 1);
      mma_phase<T, TL, true, true, true>(ws, k_i, v_im1, sacc, pfr, mprev, mu, c, lane);
      if (!lead) {
        // Steady steps issue whole copy sets, so all but the most recent one
        // are complete once no more than one set's instructions are pending.
        if (G1A3) wait_vmem_n<Copies<TL>::MIN_ISSUED>();
        else wait_vmem();
      }
      __syncthreads();
      if (DEEP && lead) wait_vmem();
      const int j = i + ahead;  // compile-time slots only occur with ahead 2 or 3 (DEEP)
      const int rj = (!lead && G1A3) ? (R + 3) % NS : (R + 2) % NS;
      lds_t* const k_j = R >= 0 ? ring.base + rj * TL::K_TILE : ring.k(j);
      lds_t* const v_jm1 = R >= 0 ? vbase + ((rj + NS - 1) % NS) * TL::V_TILE : ring.v(j - 1);
      cp.k.issue(kh + (long long)(j * BN) * kss, k_j, qw);
      cp.v.issue(vh + (long long)((j - 1) * BN) * vss, v_jm1, qw);
      softmax_tail<T, TL, false, CAUSAL, true>(ws, alpha, any, sacc, pfr, mprev, mu, i * BN, klg, thr,
                                               psum_max, lane);
      if (!DEEP && lead) wait_vmem();
      __syncthreads();
    };
    int i0 = 1;
    if (DEEP && TL::STAGES == 3) {
      for (; i0 + 2 <= steady; i0 += 3) {
        steady_step(i0, IntC<1>());
        steady_step(i0 + 1, IntC<2>());
        steady_step(i0 + 2, IntC<0>());
      }
    } else if (DEEP && TL::STAGES == 2) {
      for (; i0 + 1 <= steady; i0 += 2) {
        steady_step(i0, IntC<1>());
        steady_step(i0 + 1, IntC<0>());
      }
    }
    for (int i = i0; i <= steady; ++i) steady_step(i, IntC<-1>());
    for (int i = steady + 1 > 1 ? steady + 1 : 1; i < ntg; ++i)
      step(i, [&]() { copy_set(i + ahead); }, masked(i));
    // Step ntg: P·V of the last tile.
    ATTN_MPHASE(ntg, false, true);
  }
  if (grp == 0) __syncthreads();  // group 1 has one barrier fewer to go
  __syncthreads();
  if (KSPLIT) {
    // Group 1 may have one tile fewer (or none): it idles through the slots
    // group 0 still needs, so both pass the same barriers.
    for (int i = ntg; i < nt0; ++i) {
      __syncthreads();
      __syncthreads();
    }
    merge_key_halves<TL>(ws, smem, grp, qw, lane);
  }
  // Every ring read of this item is over (the barriers above), and Q is no
  // longer needed: the next item's prologue goes out ahead of this item's
  // stores.
  int nxt = -1;
  if (!CAUSAL && next >= 0) {
    const ItemGeom gn = item_geom<TL, CAUSAL>(p, next, grp, qw, lr);
    item_prologue<TL>(p, cp, gn, ring, ws, qw, lane);
    nxt = 0;
  }
  if (KSPLIT && grp == 1) return nxt;  // group 0 stores the merged rows
  store_output<T, TL>(p, ws, smem, sp * p.o_split + b * p.o_sb + h * p.o_sh,
                     sp * p.lse_split + (long long)bh * p.Sq, qt, qw, lane);
  const bool full_rows = qt * TL::BM + (qw * QB + QB) * 32 <= p.Sq;  // wave-uniform
  return nxt < 0 ? -1 : (full_rows ? NST : 0);
}
#undef ATTN_MPHASE
#undef ATTN_VPHASE


template <class T, class TL, bool CAUSAL>
__global__ __launch_bounds__(TL::NT) __attribute__((amdgpu_waves_per_eu(TL::WPE, TL::WPE)))
void attn_fwd_kernel(Params p) {
  __shared__ __attribute__((aligned(1024))) char smem_raw[TL::LDS_BYTES];
  lds_t* smem = (lds_t*)smem_raw;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int lane = threadIdx.x & 63;
  const int G = gridDim.x;
  Copies<TL> cp;
  const int cw = TL::KSPLIT ? (wave & 3) : wave;  // index among the waves sharing a K/V stream
  cp.k.init(cw, lane, (uint32_t)p.k_ss * 2u);
  cp.v.init(cw, lane, (uint32_t)p.v_ss * 2u);
  // Persistent loop over work items ("B200 Attention Kernel from Scratch to
  // Near-SOTA in 60 Diagrams", Chapter 14 - Persistent: a static grid-stride
  // assignment).  Workgroups are dispatched round-robin over the 8 XCDs, so
  // with xcd_remap the items of one round are renumbered to give each XCD a
  // contiguous run of items, i.e. the query tiles of the same heads, whose
  // K/V then stay in that XCD's L2.
  auto item_of = [&](int base) {
    return p.xcd_remap ? base + (int)(blockIdx.x & 7) * (G >> 3) + (int)(blockIdx.x >> 3)
                       : base + (int)blockIdx.x;
  };
  WaveState<TL> ws;
  int pre = -1;
  for (int round = 0;; ++round) {
    const int base = round * G;
    if (base >= p.n_items) break;
    const int item = item_of(base);
    const int next = (!CAUSAL && base + G < p.n_items && item_of(base + G) < p.n_items)
                         ? item_of(base + G) : -1;
    if (item < p.n_items) pre = process_item<T, TL, CAUSAL>(p, cp, smem, item, next, wave, lane, ws, pre);
  }
}

}  // namespace attn
