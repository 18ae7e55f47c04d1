// attn.hip -- causal GQA prefill and varlen SDPA for MI355X (gfx950, CDNA4).
//
// Flash-style attention: one pass over the keys with a streaming softmax
// (fp32 row sums, fp32 accumulators), bf16 MFMA for both contractions, K/V
// tiles staged through LDS and shared by every query head of a GQA group.
// The operation is defined in "[CUDA] Use Triton TMA for long-context causal
// prefill" (Summary) and "[executorch][cuda] Add a length-aware Triton SDPA
// over per-sequence KV columns" (description); the C ABI is declared in
// include/attn.h.
//
// Softmax: the first key tile of a range fixes each row's reference (its
// exact maximum over that tile) and later tiles take exponentials against
// it, with no per-tile maxima and no rescales.  Softmax does not depend on
// the reference, so this is exact while nothing overflows or underflows;
// every row checks its sum afterwards, and a workgroup with a row outside
// [2^-64, 2^64] redoes its range with the exact running maximum.  The D = 128
// prefill kernel also moves a row's reference up, exactly, on every third
// tile when its sum has passed 2^16, so that logits rising along the keys
// stay in range.
//
// Work decomposition (D = 64, 128: one workgroup = 8 waves = 256 query rows):
//   rows of a workgroup = (query heads of one KV head) x (query positions);
//   each wave owns 32 rows and keeps Q, the output accumulator, the row
//   reference and the running sum in registers for the whole key range.
//   Waves 0-3 and 4-7 form two groups that alternate MFMA and softmax phases
//   one phase apart (one wave of each group per SIMD).  Keys stream in tiles
//   of 64 through three LDS stages each of K and V, both in their natural
//   [key][d] order with XOR-swizzled 16-byte chunks.  D = 256 has its own
//   kernel of 4 waves (one per SIMD) over two stages.
//
// MFMA layout (v_mfma_f32_32x32x16_bf16): the score tile is computed
// transposed, S^T = K Q^T (keys x rows), so each lane holds 16 scores of ONE
// query row: row sums are in-lane plus a single exchange between lanes l and
// l+32.  The same registers, rounded to bf16, are directly the B operand of
// O^T = V^T P^T; the V^T operand comes from the [key][d] tile through the
// transposing LDS read (ds_read_b64_tr_b16), with the key order inside each
// 16-key group matched to which keys each lane holds.
#include <hip/hip_runtime.h>

#include <math.h>
#include <stdarg.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#include <algorithm>
#include <mutex>
#include <type_traits>
#include <utility>
#include <vector>

#include "attn.h"

// Split partials of attn_causal_prefill_noalloc: a library-owned buffer for
// callers that cannot allocate.  Host code never uses this name as an
// address (in host code it is only a stand-in for the device symbol): the
// device address comes from hipGetSymbolAddress, once per device.
static __device__ __align__(256) unsigned char scratch[ATTN_NOALLOC_SCRATCH_BYTES];

namespace {

typedef uint16_t u16;
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));

constexpr int kWave = 64;
constexpr int kWaves = 8;      // two groups of four: one wave of each group per SIMD
constexpr int kCopyWaves = 8;  // waves that issue the K/V tile copies
constexpr int kThreads = kWave * kWaves;
constexpr int kNT = 1;                  // 32-row MFMA tiles of query rows per wave
constexpr int kBM = kWaves * 32 * kNT;  // query rows per workgroup
constexpr int kBN = 64;           // keys per tile
constexpr int kMaxSplits = 16;    // key splits of a prefill launch
constexpr int kMaxVarlenSplits = 16;  // key splits of one varlen q-block
constexpr int kVarlenSplitKeys = 512; // varlen: finest target keys per split of a q-block
constexpr int kMaxLongSplits = 8;
constexpr float kLog2e = 1.4426950408889634f;

// Rows of a workgroup: Gc query heads (of one GQA group) x P positions.
struct RowMap {
    int Gc, P, hchunks;
};

__host__ __device__ inline RowMap row_map(int g, int bm = kBM) {
    RowMap r;
    r.Gc = g < bm ? g : bm;
    r.P = bm / r.Gc;
    r.hchunks = (g + r.Gc - 1) / r.Gc;
    return r;
}


// ---------------------------------------------------------------- device helpers

__device__ inline uint4 ld16(const u16* p) { return *reinterpret_cast<const uint4*>(p); }

__device__ inline bf16x8 lds_frag(const u16* p) {
    return __builtin_bit_cast(bf16x8, *reinterpret_cast<const uint4*>(p));
}

typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));

// Two floats to a packed bf16 pair, round-to-nearest-even (v_cvt_pk_bf16_f32).
__device__ inline uint32_t pack_bf16x2(float a, float b) {
    f32x2 v = {a, b};
    return __builtin_bit_cast(uint32_t, __builtin_convertvector(v, bf16x2));
}

// Key/value rows of a flat [.., L, D] tensor.
struct KVFlat {
    const u16* kb;
    const u16* vb;
    int64_t ks, vs;  // row strides in elements
};

// n mod R for n < 2^31, R >= 1, with magic = (2^32 - 1) / R: the quotient
// estimate umulhi(n, magic) is the true quotient or one less, so one
// conditional subtraction finishes (no division instruction).
__device__ inline unsigned mod_magic(unsigned n, unsigned R, unsigned magic) {
    const unsigned r = n - __umulhi(n, magic) * R;
    return r >= R ? r - R : r;
}

// Key/value rows of one column of a [rows, cols, H, D] store; position k
// lives at row k mod R.
struct KVRing {
    const u16* kb;
    const u16* vb;
    int64_t ks, vs;
    int R;
    unsigned magic;  // (2^32 - 1) / R, for mod_magic
    __device__ const u16* krow_at(int r) const { return kb + (int64_t)r * ks; }
};

// LDS tiles hold K and V in their natural [key][d] order, 16-byte chunks of
// each row XOR-swizzled so that the MFMA operand reads (ds_read_b128 for K,
// ds_read_b64_tr_b16 for V) hit distinct banks.  Chunk c of row r sits at
// position c ^ swz(r).
template <int D>
__device__ __host__ constexpr int swz(int r) {
    // D = 256 rows (512 bytes) start on the same bank as D = 128 rows, so
    // they take the same pattern on the low four chunk bits
    return D >= 128 ? (((r & 3) << 2) | ((r >> 2) & 3)) : ((((r >> 1) & 1) << 2) | ((r >> 2) & 3));
}

typedef __attribute__((address_space(3))) void lds_void;
typedef __attribute__((address_space(1))) const void glb_void;

// Geometry of the global -> LDS tile copies.  Each wave instruction fills
// 1 KB of LDS: lane l's 16 bytes land at chunk position (instruction * 64 + l),
// which holds logical chunk (position ^ swz(row)) of its row.  Wave w issues
// instructions w, w + NW, ...
template <int D, int NW = kCopyWaves>
struct CopyPlan {
    static constexpr int CH = D / 8;                // 16-byte chunks per row
    static constexpr int ROWS = 64 / CH;            // rows per wave instruction
    static constexpr int INSTR = kBN / ROWS;        // wave instructions per tensor
    static constexpr int PER_WAVE = INSTR / NW;
    static __device__ int wave() { return __builtin_amdgcn_readfirstlane(threadIdx.x / kWave); }
    static __device__ int row(int i) {
        return (wave() + i * NW) * ROWS + (threadIdx.x & (kWave - 1)) / CH;
    }
    static __device__ int chunk(int i) {
        return ((threadIdx.x & (kWave - 1)) % CH) ^ swz<D>(row(i));
    }
    static __device__ int lds_off(int i) {  // elements
        return (wave() + i * NW) * 512;
    }
};

// Per-lane byte offsets of this wave's copy instructions inside a tile of
// consecutive rows (row * stride + chunk), the same for every tile.
template <int D, int NW = kCopyWaves>
struct CopyOffsets {
    uint32_t o[CopyPlan<D, NW>::PER_WAVE];
};

template <int D, int NW = kCopyWaves>
__device__ inline CopyOffsets<D, NW> copy_offsets(int rs2) {
    typedef CopyPlan<D, NW> CP;
    CopyOffsets<D, NW> c;
#pragma unroll
    for (int i = 0; i < CP::PER_WAVE; ++i) c.o[i] = (uint32_t)(CP::row(i) * rs2 + 16 * CP::chunk(i));
    return c;
}

// r mod R for the rows r of this wave's copy instructions inside a tile
// (ring storage of R rows).
template <int D>
__device__ inline CopyOffsets<D> ring_offsets(int R) {
    CopyOffsets<D> c;
#pragma unroll
    for (int i = 0; i < CopyPlan<D>::PER_WAVE; ++i)
        c.o[i] = (uint32_t)CopyPlan<D>::row(i) % (uint32_t)R;
    return c;
}

#if defined(__HIP_DEVICE_COMPILE__)
typedef __amdgpu_buffer_rsrc_t BufRsrc;
#else
struct BufRsrc {  // placeholder: buffer resources exist only in the device pass
    int w[4];
};
#endif

// This wave's share of the global -> LDS copy of keys [k0, k0 + kBN) of one
// tensor (K or V) of flat storage, prepared with scalar work and issued one
// instruction at a time, without branches, so that the instructions can sit
// between MFMAs.  The copy goes through a buffer resource spanning exactly
// the rows below k_hi: rows past it, and every row of a tile at or past
// k_hi (whose stage nobody reads), land in LDS as zeros and touch no memory.
template <int D, int NW = kCopyWaves>
struct TileCopyFlat {
    static constexpr int N = CopyPlan<D, NW>::PER_WAVE;
    BufRsrc r;
    u16* dst;
    const uint32_t* o;
    __device__ TileCopyFlat(const KVFlat&, const u16* tb, int64_t rs, int rs2,
                            const CopyOffsets<D, NW>& co, int k0, int k_hi, u16* d)
        : dst(d), o(co.o) {
        // 32-bit scalar arithmetic, no branches (k0 <= k_hi)
        const int nv = min(k_hi - k0, kBN);
        const uint32_t nrec = nv > 0 ? (uint32_t)((nv - 1) * rs2 + 2 * D) : 0u;
#if defined(__HIP_DEVICE_COMPILE__)
        r = __builtin_amdgcn_make_buffer_rsrc((void*)(tb + (int64_t)(nv > 0 ? k0 : 0) * rs), 0,
                                              nrec, 0x00020000);
#else
        (void)tb, (void)rs, (void)nrec;
#endif
    }
    __device__ void issue(int i) const {
#if defined(__HIP_DEVICE_COMPILE__)
        __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (lds_void*)(dst + CopyPlan<D, NW>::lds_off(i)),
                                                 16, o[i], 0, 0, 0);
#else
        (void)i;
#endif
    }
};

// The same for one column of ring storage: each lane addresses its own row
// (position mod R), so a tile may wrap the ring.  Rows past k_hi repeat row
// k_hi - 1, and a tile at or past k_hi copies row k_hi - 1 throughout.
//   The store row of key kc + r is (kc mod R + r mod R) mod R: kc mod R and
//   (for the clamped rows) last mod R are uniform, taken once per tile with
//   mod_magic; r mod R of this lane's copy rows comes in `co` (ring_offsets),
//   so each copy adds and subtracts R at most once, with no division.
template <int D>
struct TileCopyRing {
    static constexpr int N = CopyPlan<D>::PER_WAVE;
    const u16* tb;
    int64_t rs;
    int R, base, last, lastm;
    const uint32_t* o;
    u16* dst;
    __device__ TileCopyRing(const KVRing& kv, const u16* t, int64_t s, int, const CopyOffsets<D>& co,
                            int k0, int k_hi, u16* d)
        : tb(t), rs(s), R(kv.R), o(co.o), dst(d) {
        const int kc = k0 < k_hi ? k0 : k_hi - 1;
        last = k_hi - 1 - kc;
        base = (int)mod_magic((unsigned)kc, (unsigned)R, kv.magic);
        lastm = (int)mod_magic((unsigned)last, (unsigned)R, kv.magic);
    }
    __device__ void issue(int i) const {
        const int r = CopyPlan<D>::row(i);
        unsigned row = (unsigned)base + (r < last ? o[i] : (unsigned)lastm);
        row = row >= (unsigned)R ? row - (unsigned)R : row;
        __builtin_amdgcn_global_load_lds(
            (glb_void*)(tb + (int64_t)row * rs + 8 * CopyPlan<D>::chunk(i)),
            (lds_void*)(dst + CopyPlan<D>::lds_off(i)), 16, 0, 0);
    }
};

template <int D, class KV>
struct TileCopySel;
template <int D>
struct TileCopySel<D, KVFlat> {
    typedef TileCopyFlat<D> T;
};
template <int D>
struct TileCopySel<D, KVRing> {
    typedef TileCopyRing<D> T;
};

// No copy (an MFMA region without copies).
struct NoCopy {
    static constexpr int N = 0;
    __device__ void issue(int) const {}
};

// Positions of the copy instructions among the NM MFMAs of a region: copy j
// of NC follows MFMA slot(j), spread evenly.
__device__ __host__ constexpr int copy_slot(int j, int NC, int NM) {
    return j * NM / NC + NM / (2 * NC);
}

// Wait for this wave's outstanding global -> LDS copies, then for every wave.
__device__ inline void tile_barrier() {
    __builtin_amdgcn_s_waitcnt(0x0F70);  // vmcnt(0)
    __builtin_amdgcn_s_barrier();
}

// Workgroup barrier between ping-pong phases; no instruction is scheduled
// across it, so MFMA and VALU work stay in their phases.
__device__ inline void phase_barrier() {
    __builtin_amdgcn_sched_barrier(0);
    __builtin_amdgcn_s_barrier();
    __builtin_amdgcn_sched_barrier(0);
}

typedef short s16x4 __attribute__((ext_vector_type(4)));

// V^T operand of O^T += V^T P^T for d-tile dt and key chunk c4: lane l needs
// V[key(l)][32*dt + l%32] for its 8 key slots; two transposing reads give 4
// keys each (lanes 4j..4j+3 of a 16-lane group point at key j's 4 d values).
template <int D>
__device__ inline bf16x8 v_frag(const u16* Vs, int dt, int c4, int lane) {
    constexpr int CH = D / 8;
    const int h = lane >> 5, dh = (lane >> 4) & 1, L = lane & 15;
    const int j = L >> 2, q = L & 3;
    const int c = 4 * dt + 2 * dh + (q >> 1);
    const int r0 = 16 * c4 + 4 * h + j, r1 = r0 + 8;
    const u16* p0 = Vs + r0 * D + 8 * (c ^ swz<D>(r0)) + 4 * (q & 1);
    const u16* p1 = Vs + r1 * D + 8 * (c ^ swz<D>(r1)) + 4 * (q & 1);
    (void)CH;
    s16x4 a = __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) s16x4*)p0);
    s16x4 b = __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) s16x4*)p1);
    typedef long long i64x2 __attribute__((ext_vector_type(2)));
    i64x2 ab = {__builtin_bit_cast(long long, a), __builtin_bit_cast(long long, b)};
    return __builtin_bit_cast(bf16x8, ab);
}

// K operand of S^T = K Q^T for key subtile t and d step kk.
template <int D>
__device__ inline bf16x8 k_frag(const u16* Ks, int t, int kk, int lane) {
    const int r = 32 * t + (lane & 31), c = 2 * kk + (lane >> 5);
    return lds_frag(Ks + r * D + 8 * (c ^ swz<D>(r)));
}

__device__ inline float max_across_halves(float x) {
    auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    return __builtin_fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}

__device__ inline float sum_across_halves(float x) {
    auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

// Per-lane online-softmax state of the wave's kNT query rows held by this
// lane (lanes l and l+32 share a row).
template <int D>
struct RowState {
    f32x16 o[kNT][D / 32];  // O^T accumulators: d = 32*dt + 8*(r/4) + 4*(lane/32) + r%4
    float m[kNT];           // running maximum of the scores (-inf: nothing seen)
    float l[kNT];           // this lane's share of the running sum
    f32x16 mneg[kNT];       // -(fixed reference) in every element: the scores' initial value
};

// After the tile that fixes the references: the score MFMAs of later tiles
// start from -m (0 for a row that has seen nothing), so they yield s - m.
template <int D>
__device__ inline void set_reference(RowState<D>& st) {
#pragma unroll
    for (int nt = 0; nt < kNT; ++nt) {
        const float v = st.m[nt] == -INFINITY ? 0.f : -st.m[nt];
#pragma unroll
        for (int r = 0; r < 16; ++r) st.mneg[nt][r] = v;
    }
}

// Visible keys of one row inside the range [k_lo, k_hi): the interval
// lo .. lo + span, in int32.
struct LaneBounds {
    int lo;
    int span;
};

__device__ inline LaneBounds lane_bounds(int k_lo, int k_hi, int causal, int window,
                                         int64_t p_lane) {
    int64_t hi = k_hi - 1;
    if (causal && p_lane < hi) hi = p_lane;
    int64_t lo = k_lo;
    if (window > 0 && p_lane - window + 1 > lo) lo = p_lane - window + 1;
    LaneBounds b;
    if (hi < lo) {
        b.lo = k_hi + (1 << 20);  // every key of the range lies below lo
        b.span = 0;
    } else {
        b.lo = (int)lo;
        b.span = (int)(hi - lo);
    }
    return b;
}

// Scores of one key tile for the wave's rows: [row tile][32-key subtile].
typedef f32x16 TileScores[kNT][2];

// S^T = K Q^T for one key tile (keys in LDS).  Each K fragment read from LDS
// feeds the MFMAs of all kNT row tiles.  The copy instructions of c1 and c2
// are spread between the MFMAs.
// PRE: the accumulators start from init (the negated fixed references), so
// the tile comes out as s - m.
template <int D, class C1, class C2, bool PRE = false>
__device__ inline void qk_tile(const u16* Ks, const bf16x8 (*qf)[D / 16], TileScores& s,
                               const C1& c1, const C2& c2, const f32x16* init = nullptr) {
    const int lane = threadIdx.x & (kWave - 1);
    constexpr int NR = 2 * (D / 16), NM = 2 * kNT * (D / 16), NC = C1::N + C2::N;
#pragma unroll
    for (int nt = 0; nt < kNT; ++nt) s[nt][0] = s[nt][1] = PRE ? init[nt] : f32x16{};
#pragma unroll
    for (int kk = 0; kk < D / 16; ++kk) {
        const bf16x8 a0 = k_frag<D>(Ks, 0, kk, lane), a1 = k_frag<D>(Ks, 1, kk, lane);
#pragma unroll
        for (int nt = 0; nt < kNT; ++nt) {
            s[nt][0] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a0, qf[nt][kk], s[nt][0], 0, 0, 0);
            s[nt][1] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a1, qf[nt][kk], s[nt][1], 0, 0, 0);
        }
#pragma unroll
        for (int j = 0; j < NC; ++j) {
            const int sl = copy_slot(j, NC, NM);
            if (sl >= 2 * kNT * kk && sl < 2 * kNT * (kk + 1)) {
                if (j < C1::N)
                    c1.issue(j);
                else
                    c2.issue(j - C1::N);
            }
        }
    }
    // keep 4 fragment reads ahead of the MFMAs: LDS latency hides behind them
    __builtin_amdgcn_sched_group_barrier(0x100, 4, 0);
#pragma unroll
    for (int i = 0; i < NM; ++i) {
        __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
        if (4 + (i + 1) * NR / NM <= NR && (i + 1) * NR % NM == 0)
            __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
#pragma unroll
        for (int j = 0; j < NC; ++j)
            if (copy_slot(j, NC, NM) == i) __builtin_amdgcn_sched_group_barrier(0x010, 1, 0);
    }
}

// Scores of keys a row does not see become -inf: key k0 + 32t + 8(r/4) +
// 4hh + r%4 is visible iff 0 <= key - lo <= span.
__device__ inline void mask_tile(TileScores& s, int k0, const LaneBounds* lb) {
    const int hh = (threadIdx.x & (kWave - 1)) >> 5;
#pragma unroll
    for (int nt = 0; nt < kNT; ++nt) {
        const unsigned base = (unsigned)(k0 + 4 * hh - lb[nt].lo);
        const unsigned span = (unsigned)lb[nt].span;
#pragma unroll
        for (int t = 0; t < 2; ++t)
#pragma unroll
            for (int r = 0; r < 16; ++r) {
                const unsigned d = base + (unsigned)(32 * t + 8 * (r >> 2) + (r & 3));
                s[nt][t][r] = d <= span ? s[nt][t][r] : -INFINITY;
            }
    }
}

// Running maxima after a tile: m_new = max(m, row max of s); alpha =
// 2^((m - m_new) c) rescales what was accumulated against m (0 when nothing
// was seen before).
__device__ inline void update_max(const TileScores& s, float c, float* m, float* alpha) {
#pragma unroll
    for (int nt = 0; nt < kNT; ++nt) {
        float mq[4] = {m[nt], -INFINITY, -INFINITY, -INFINITY};  // 4 independent chains
#pragma unroll
        for (int t = 0; t < 2; ++t)
#pragma unroll
            for (int r = 0; r < 16; ++r) mq[r & 3] = __builtin_fmaxf(mq[r & 3], s[nt][t][r]);
        const float mx =
            __builtin_fmaxf(__builtin_fmaxf(mq[0], mq[1]), __builtin_fmaxf(mq[2], mq[3]));
        const float m_new = max_across_halves(mx);
        const float m_use = m_new == -INFINITY ? 0.f : m_new;  // guard: nothing visible yet
        alpha[nt] = m[nt] == -INFINITY ? 0.f : __builtin_amdgcn_exp2f((m[nt] - m_use) * c);
        m[nt] = m_new;
    }
}

// P = 2^(s c - m c) rounded to packed bf16 pairs (the B operand of the PV
// MFMA), and the row sums of P.  Masked scores are -inf and c > 0, so they
// give exactly 0.  The sums use plain adds: the packed dot product would wait
// on the matrix core while the partner wave's MFMAs run.
//
// Which values the sums add: with a fixed reference the largest weight of a
// row is not 1, so its bf16 rounding (up to 2^-9 of itself) moves the output
// by up to 2^-9 of a V value when one key dominates, on top of the output's
// own rounding.  Adding the rounded weights (RS) makes the normalizer the sum
// of the weights the PV product used, and that error cancels.  It costs two
// VALU instructions per pair, 2.4-5.6 % of a prefill call with the scale in
// Q.  So the fixed-reference pass takes it where the softmax can be sharper
// than at the standard scale (exact Q: |scale| above 1/sqrt(D); varlen,
// where it measured free) and keeps the unrounded sums with the scale in Q;
// the exact pass, which redoes a whole range when needed, always takes it.
typedef uint32_t TileP[kNT][2][8];

// PRE: s already holds s - m (qk_tile from the negated references), and
// c = 1, so P = 2^s.  RS: the sums add the rounded weights.
template <bool PRE = false, bool RS = true>
__device__ inline void softmax_tile(const TileScores& s, float c, const float* m, TileP& pk,
                                    float* lsum) {
#pragma unroll
    for (int nt = 0; nt < kNT; ++nt) {
        const float mc = (m[nt] == -INFINITY ? 0.f : m[nt]) * c;  // reference 0 before any key
        float ls[4] = {0.f, 0.f, 0.f, 0.f};  // 4 independent chains
#pragma unroll
        for (int t = 0; t < 2; ++t)
#pragma unroll
            for (int r = 0; r < 16; r += 2) {
                const float x0 = __builtin_amdgcn_exp2f(PRE ? s[nt][t][r] : fmaf(s[nt][t][r], c, -mc));
                const float x1 =
                    __builtin_amdgcn_exp2f(PRE ? s[nt][t][r + 1] : fmaf(s[nt][t][r + 1], c, -mc));
                const uint32_t p2 = pack_bf16x2(x0, x1);  // element 0 in the low half
                pk[nt][t][r >> 1] = p2;
                ls[(r >> 1) & 3] += RS ? __uint_as_float(p2 << 16) : x0;
                ls[(r >> 1) & 3] += RS ? __uint_as_float(p2 & 0xffff0000u) : x1;
            }
        lsum[nt] = (ls[0] + ls[1]) + (ls[2] + ls[3]);
    }
}

// O^T += V^T P^T for one key tile (V in LDS), 16 keys per MFMA; each V
// fragment feeds the MFMAs of all kNT row tiles.  The copy instructions of
// c1 are spread between the MFMAs.
template <int D, class C1>
__device__ inline void pv_tile(const u16* Vs, const TileP& pk, RowState<D>& st, const C1& c1) {
    const int lane = threadIdx.x & (kWave - 1);
    constexpr int NF = (kBN / 16) * (D / 32);  // fragments, 2 reads each
    constexpr int NC = C1::N;
#pragma unroll
    for (int c4 = 0; c4 < kBN / 16; ++c4) {
#pragma unroll
        for (int dt = 0; dt < D / 32; ++dt) {
            const bf16x8 vf = v_frag<D>(Vs, dt, c4, lane);
#pragma unroll
            for (int nt = 0; nt < kNT; ++nt) {
                const uint32_t* w = &pk[nt][c4 >> 1][4 * (c4 & 1)];
                const bf16x8 pb = __builtin_bit_cast(bf16x8, make_uint4(w[0], w[1], w[2], w[3]));
                st.o[nt][dt] =
                    __builtin_amdgcn_mfma_f32_32x32x16_bf16(vf, pb, st.o[nt][dt], 0, 0, 0);
            }
            const int f = c4 * (D / 32) + dt;
#pragma unroll
            for (int j = 0; j < NC; ++j)
                if (copy_slot(j, NC, NF) == f) c1.issue(j);
        }
    }
    // keep 4 fragments (8 transposing reads) ahead of the MFMAs
    __builtin_amdgcn_sched_group_barrier(0x100, 8, 0);
#pragma unroll
    for (int f = 0; f < NF; ++f) {
#pragma unroll
        for (int nt = 0; nt < kNT; ++nt) __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
        if (f + 4 < NF) __builtin_amdgcn_sched_group_barrier(0x100, 2, 0);
#pragma unroll
        for (int j = 0; j < NC; ++j)
            if (copy_slot(j, NC, NF) == f) __builtin_amdgcn_sched_group_barrier(0x010, 1, 0);
    }
}

// pv_tile for the previous key tile, then qk_tile for this one, as one
// software pipeline: every MFMA is followed by the fragment reads of the
// MFMA AHEAD places later, across the boundary between the two products, so
// the scores do not start with an LDS round trip.  Copies of cp spread
// through the PV MFMAs, those of cq through the score MFMAs.
template <int D, class CP, class CQ, bool PRE>
__device__ inline void pv_qk_tile(const u16* Vs, const u16* Ks, const bf16x8 (*qf)[D / 16],
                                  const TileP& pk, TileScores& s, RowState<D>& st, const CP& cp,
                                  const CQ& cq, const f32x16* init) {
    static_assert(kNT == 1, "one MFMA per fragment");
    const int lane = threadIdx.x & (kWave - 1);
    constexpr int NF = (kBN / 16) * (D / 32);  // PV fragments, 2 reads each
    constexpr int NK = 2 * (D / 16);           // K fragments, 1 read each
    constexpr int AHEAD = 2;  // measured better than 3 or 4 at D=128
#pragma unroll
    for (int c4 = 0; c4 < kBN / 16; ++c4) {
#pragma unroll
        for (int dt = 0; dt < D / 32; ++dt) {
            const bf16x8 vf = v_frag<D>(Vs, dt, c4, lane);
            const uint32_t* w = &pk[0][c4 >> 1][4 * (c4 & 1)];
            const bf16x8 pb = __builtin_bit_cast(bf16x8, make_uint4(w[0], w[1], w[2], w[3]));
            st.o[0][dt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(vf, pb, st.o[0][dt], 0, 0, 0);
            const int f = c4 * (D / 32) + dt;
#pragma unroll
            for (int j = 0; j < CP::N; ++j)
                if (copy_slot(j, CP::N, NF) == f) cp.issue(j);
        }
    }
    s[0][0] = s[0][1] = PRE ? init[0] : f32x16{};
#pragma unroll
    for (int kk = 0; kk < D / 16; ++kk) {
        const bf16x8 a0 = k_frag<D>(Ks, 0, kk, lane), a1 = k_frag<D>(Ks, 1, kk, lane);
        s[0][0] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a0, qf[0][kk], s[0][0], 0, 0, 0);
        s[0][1] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a1, qf[0][kk], s[0][1], 0, 0, 0);
#pragma unroll
        for (int j = 0; j < CQ::N; ++j) {
            const int sl = copy_slot(j, CQ::N, NK);
            if (sl >= 2 * kk && sl < 2 * (kk + 1)) cq.issue(j);
        }
    }
    // MFMA i (PV for i < NF, scores after) is followed by the reads of MFMA
    // i + AHEAD: two transposing reads for a V fragment, one for a K fragment
    __builtin_amdgcn_sched_group_barrier(0x100, 2 * AHEAD, 0);
#pragma unroll
    for (int i = 0; i < NF + NK; ++i) {
        __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
        const int g = i + AHEAD;
        if (g < NF)
            __builtin_amdgcn_sched_group_barrier(0x100, 2, 0);
        else if (g < NF + NK)
            __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
#pragma unroll
        for (int j = 0; j < CP::N; ++j)
            if (i < NF && copy_slot(j, CP::N, NF) == i) __builtin_amdgcn_sched_group_barrier(0x010, 1, 0);
#pragma unroll
        for (int j = 0; j < CQ::N; ++j)
            if (i >= NF && copy_slot(j, CQ::N, NK) == i - NF)
                __builtin_amdgcn_sched_group_barrier(0x010, 1, 0);
    }
}

template <int D>
__device__ inline void rescale(const float* alpha, RowState<D>& st) {
#pragma unroll
    for (int nt = 0; nt < kNT; ++nt) {
        st.l[nt] *= alpha[nt];
        if (__any(alpha[nt] != 1.f)) {
#pragma unroll
            for (int dt = 0; dt < D / 32; ++dt) st.o[nt][dt] *= alpha[nt];
        }
    }
}

// LDS of one workgroup: three stages of K and V tiles.
template <int D>
struct TileSmem {
    u16* k[3];
    u16* v[3];
    int* rerun;  // set when the fixed-reference pass must be redone exactly
};

// LDS tile (32 rows x D) of wave w for the row stores: half of a K or V
// stage, which no wave reads once the key range is done.
template <int D>
__device__ inline u16* row_tile(const TileSmem<D>& sm, int w) {
    const int i = w >> 1;
    u16* const st = i == 0 ? sm.k[0] : i == 1 ? sm.v[0] : i == 2 ? sm.k[1] : sm.v[1];
    return st + (w & 1) * 32 * D;
}

// Per-range constants of the key loop.
template <int D, class KV>
struct KeyLoop {
    KV kv;
    int k_lo, k_hi;
    int n;                     // tiles in the range
    int ks2, vs2;              // row strides in bytes (flat storage: below 2^25)
    CopyOffsets<D> kco, vco;   // per-lane copy offsets (full tiles)
    int t_in0, t_in1;          // tiles t_in0 <= t < t_in1 need no mask
    __device__ int k0(int t) const { return k_lo + t * kBN; }
    // first key of a copied tile: k_hi for tiles past the range (nothing to copy)
    __device__ int k0c(int t) const { return t < n ? k_lo + t * kBN : k_hi; }
    // a tile straddles a causal, window or range edge of some row
    __device__ bool needs_mask(int t) const { return t < t_in0 || t >= t_in1; }
};

// Tiles of [k_lo, k_hi) that need no mask: every key of the tile lies below
// k_hi, at or before the smallest row position (causal) and past the window
// start of the largest.
template <int D, class KV>
__device__ inline void interior_tiles(KeyLoop<D, KV>& L, int causal, int window, int64_t p_min,
                                      int64_t p_max) {
    const int n = (L.k_hi - L.k_lo + kBN - 1) / kBN;
    int64_t t1 = (L.k_hi - L.k_lo) / kBN;  // full tiles
    if (causal) {
        // k_lo + t*kBN + kBN - 1 <= p_min
        const int64_t c = p_min - L.k_lo - (kBN - 1);
        const int64_t tc = c < 0 ? 0 : c / kBN + 1;
        if (tc < t1) t1 = tc;
    }
    int64_t t0 = 0;
    if (window > 0) {
        // k_lo + t*kBN > p_max - window
        const int64_t w = p_max - window - L.k_lo;
        t0 = w < 0 ? 0 : w / kBN + 1;
    }
    if (t1 > n) t1 = n;
    if (t0 > t1) t0 = t1;
    L.t_in0 = (int)t0;
    L.t_in1 = (int)t1;
}

// Pin the values that cross a phase boundary: an empty asm that reads and
// rewrites them keeps their producers before it and their consumers after
// it, so no pass moves MFMA or VALU work into the other phase.
__device__ inline void pin(f32x16& x) { asm volatile("" : "+v"(x)); }
__device__ inline void pin(uint32_t& x) { asm volatile("" : "+v"(x)); }
__device__ inline void pin(float& x) { asm volatile("" : "+v"(x)); }

template <int D>
__device__ inline void pin_m_outputs(TileScores& S, RowState<D>& st, bool qk, bool pv) {
#pragma unroll
    for (int nt = 0; nt < kNT; ++nt) {
        if (qk) {
            pin(S[nt][0]);
            pin(S[nt][1]);
        }
        if (pv)
#pragma unroll
            for (int dt = 0; dt < D / 32; ++dt) pin(st.o[nt][dt]);
    }
}

template <int D>
__device__ inline void pin_v_outputs(TileP& pk, RowState<D>& st) {
#pragma unroll
    for (int nt = 0; nt < kNT; ++nt) {
#pragma unroll
        for (int t = 0; t < 2; ++t)
#pragma unroll
            for (int r = 0; r < 8; ++r) pin(pk[nt][t][r]);
        pin(st.m[nt]);
        pin(st.l[nt]);
    }
}

// MFMA phase of a wave: O += P(k-1) V(k-1) (V in Vs) and S(k) = K(k) Q^T (K
// in Ks), with this wave's copies of a later K tile (ck) spread through the
// PV product and of a later V tile (cv) through the scores.  No VALU work,
// so the MFMAs issue back to back.
template <int D, bool QK, bool PV, bool PRE, class CK, class CV>
__device__ inline void m_phase(const u16* Ks, const u16* Vs, const bf16x8 (*qf)[D / 16],
                               TileScores& S, const TileP& pk, RowState<D>& st, const CK& ck,
                               const CV& cv) {
    if (PV && QK && D >= 128 && PRE) {
        pv_qk_tile<D, CK, CV, PRE>(Vs, Ks, qf, pk, S, st, ck, cv, st.mneg);
    } else {
        // D=64, and varlen's short items, measured faster with the two
        // products as separate scheduling regions
        if (PV) pv_tile<D>(Vs, pk, st, ck);
        if (PV && QK) __builtin_amdgcn_sched_barrier(0);
        if (QK) qk_tile<D, CV, NoCopy, PRE>(Ks, qf, S, cv, NoCopy{}, st.mneg);
    }
    pin_m_outputs<D>(S, st, QK, PV);
}

// Refresh of the fixed references in the fixed-reference pass when the
// scores come out of the MFMAs relative to them (scale in Q): on every
// third tile, before its P, a row whose running sum lies in (2^16, 2^64]
// moves its reference up by d = floor(log2 l).  Its l and O are multiplied
// by 2^-d, which is exact (a power of two), the current tile's scores lose
// d, and later tiles start from the new reference.  Softmax does not depend
// on the reference, so this changes only the range: when the logits rise
// along the keys (by up to about 0.2 in log2 units per key on average over
// three tiles), the sums stay below 2^64 instead of overflowing it, which
// would send the workgroup to the pass with the exact running maximum.  A
// row above 2^64 is left alone (its P may already have lost range), so the
// check after the pass still sees it: a sum only grows between refreshes.
// Sums that are too small need nothing: they only grow, and the terms that
// underflowed are negligible next to a final sum of at least 2^-64.  A wave
// with no lane share above 2^16 pays a compare.
constexpr float kRefreshHi = 0x1p16f;
// D = 64: more VALU work beside the partner wave's MFMA phase lengthens that
// phase, which bounds the step there; D = 256 runs its own loop
template <int D>
constexpr bool kRefresh = D == 128;

template <int D>
__device__ inline void refresh_reference(TileScores& s, RowState<D>& st) {
    bool out = false;
#pragma unroll
    for (int nt = 0; nt < kNT; ++nt) out |= st.l[nt] > kRefreshHi;
    if (__builtin_expect(!__any(out), 1)) return;
#pragma unroll
    for (int nt = 0; nt < kNT; ++nt) {
        const float lrow = sum_across_halves(st.l[nt]);
        const bool move = lrow > kRefreshHi && lrow <= 0x1p64f;
        // floor(log2 lrow) from the exponent field, 16 <= d <= 64
        const int d = move ? __builtin_amdgcn_frexp_expf(lrow) - 1 : 0;
        const float df = (float)d;
#pragma unroll
        for (int t = 0; t < 2; ++t)
#pragma unroll
            for (int r = 0; r < 16; ++r) s[nt][t][r] -= df;
        const float ref = (st.m[nt] == -INFINITY ? 0.f : st.m[nt]) + df;
        st.m[nt] = move ? ref : st.m[nt];
#pragma unroll
        for (int r = 0; r < 16; ++r) st.mneg[nt][r] = move ? -ref : st.mneg[nt][r];
        st.l[nt] = __builtin_amdgcn_ldexpf(st.l[nt], -d);
#pragma unroll
        for (int dt = 0; dt < D / 32; ++dt)
#pragma unroll
            for (int r = 0; r < 16; ++r)
                st.o[nt][dt][r] = __builtin_amdgcn_ldexpf(st.o[nt][dt][r], -d);
    }
}

// VALU phase of a wave for tile k: mask (edge tiles), then P(k) and its row
// sums.  EXACT: against each row's running maximum, with the rescale of O
// and l when it moves.  Otherwise against the row's fixed reference st.m (0
// while it is -inf), with no maxima and no rescale; the caller checks
// afterwards that every row's sum stayed in range.
template <int D, bool EXACT, bool PRE, class KV, bool REF = false, bool RS = true>
__device__ inline void v_phase(const KeyLoop<D, KV>& L, int k, float c, const LaneBounds* lb,
                               TileScores& S, TileP& pk, RowState<D>& st) {
    if (L.needs_mask(k)) mask_tile(S, L.k0(k), lb);
    if (REF && PRE && !EXACT) refresh_reference<D>(S, st);
    if (EXACT) {
        float alpha[kNT];
        update_max(S, c, st.m, alpha);
        rescale<D>(alpha, st);
    }
    float lsum[kNT];
    softmax_tile<PRE, RS>(S, c, st.m, pk, lsum);
#pragma unroll
    for (int nt = 0; nt < kNT; ++nt) st.l[nt] += lsum[nt];
    pin_v_outputs<D>(pk, st);
}

// End of an MFMA phase: wait until at most NPEND of this wave's copies are
// in flight (those issued in this phase), then the workgroup barrier.
template <int NPEND>
__device__ inline void copy_wait_barrier() {
    // vmcnt is 6 bits: 3:0 and 15:14 of the immediate
    static_assert(NPEND >= 0 && NPEND < 64, "vmcnt field");
    __builtin_amdgcn_sched_barrier(0);
    __builtin_amdgcn_s_waitcnt(0x0F70 | (NPEND & 15) | ((NPEND >> 4) << 14));
    __builtin_amdgcn_s_barrier();
    __builtin_amdgcn_sched_barrier(0);
}

template <int D, class KV>
__device__ inline typename TileCopySel<D, KV>::T k_copy(const KeyLoop<D, KV>& L, int t, u16* dst) {
    return typename TileCopySel<D, KV>::T(L.kv, L.kv.kb, L.kv.ks, L.ks2, L.kco, L.k0c(t), L.k_hi,
                                          dst);
}
template <int D, class KV>
__device__ inline typename TileCopySel<D, KV>::T v_copy(const KeyLoop<D, KV>& L, int t, u16* dst) {
    return typename TileCopySel<D, KV>::T(L.kv, L.kv.vb, L.kv.vs, L.vs2, L.vco, L.k0c(t), L.k_hi,
                                          dst);
}

// One ping-pong step for tile k >= 1: the MFMA phase M(k) (scores of tile k
// from Kr, PV of tile k-1 from Vr) with the copies ck of K(k+2) and cv of
// V(k+1), then the softmax phase of tile k, each closed by a workgroup
// barrier.  At the end of M(k) every wave waits for its copies of the
// previous step (K(k+1), V(k)); those of this step stay in flight.  The
// softmax phase also prepares the next step's copy descriptors (K(k+3) into
// Kn, V(k+2) into Vn): scalar work that would otherwise delay the first
// MFMA of the next phase.
//
// The SIMD's issue arbiter prefers the older of two ready waves, so the MFMA
// phase of group 1 (the younger waves) loses issue slots to group 0's
// softmax.  Where it measured faster, the MFMA phase runs at wave priority
// 2: column-store (varlen) loops, and D = 64, whose copy descriptors are
// then built after the barrier, which gives the partner's softmax a start
// before the prioritised MFMAs.  The D = 128 prefill loop measured slower
// with either change.
template <int D, bool EXACT, bool PRE, class KV, bool REF = false, bool RS = true>
__device__ inline void pp_step(const KeyLoop<D, KV>& L, int k, const bf16x8 (*qf)[D / 16],
                               float c, const LaneBounds* lb, TileScores& S, TileP& pk,
                               RowState<D>& st, const u16* Kr, const u16* Vr,
                               typename TileCopySel<D, KV>::T& ck,
                               typename TileCopySel<D, KV>::T& cv, u16* Kn, u16* Vn) {
    typedef typename TileCopySel<D, KV>::T TC;
    constexpr bool ring = std::is_same<KV, KVRing>::value;
    constexpr bool prio = ring || D == 64, late = !ring && D == 64;
    if (prio) {
        __builtin_amdgcn_s_setprio(2);
        __builtin_amdgcn_sched_barrier(0);
    }
    m_phase<D, true, true, PRE>(Kr, Vr, qf, S, pk, st, ck, cv);
    if (prio) {
        __builtin_amdgcn_sched_barrier(0);
        __builtin_amdgcn_s_setprio(0);
    }
    copy_wait_barrier<2 * TC::N>();
    v_phase<D, EXACT, PRE, KV, REF, RS>(L, k, c, lb, S, pk, st);
    if (!late) {
        ck = k_copy<D>(L, k + 3, Kn);
        cv = v_copy<D>(L, k + 2, Vn);
    }
    phase_barrier();
    if (late) {
        ck = k_copy<D>(L, k + 3, Kn);
        cv = v_copy<D>(L, k + 2, Vn);
    }
}

// Attend the keys [k_lo, k_hi) for the rows of this wave.
//
// Ping-pong between the two wave groups of the workgroup (waves 0-3 and
// 4-7, one of each on every SIMD): every wave alternates an MFMA phase M(k)
// (the PV product of tile k-1 and the scores of tile k) and a VALU phase
// (the softmax of tile k), with a workgroup barrier after each phase.  Group
// 1 starts one phase late, so on every SIMD one wave issues MFMAs while the
// other runs its softmax.  K and V tiles stream through three LDS stages
// each: during M(k) every wave issues its share of the copies of K(k+2) and
// V(k+1) (into the stages of K(k-1) and V(k-2), which both groups have
// finished reading), spread between its MFMAs, and at the end of M(k) waits
// for its share of K(k+1) and V(k), which the next MFMA phases read.
// Copies of tiles past the range fill unread stages.  M(0) (scores only) and
// M(n) (PV only) are peeled off the loop, which is unrolled by three so that
// every stage is a distinct LDS object.
//   p_lane[nt]: position of this lane's row in row tile nt; p_min/p_max:
//   extreme positions of the workgroup's rows (for the per-tile mask
//   decision).
template <int D, bool EXACT, bool PRE, class KV, bool RS>
__device__ void attend_range(const KV& kv, int k_lo, int k_hi, int causal, int window,
                             const int64_t* p_lane, int64_t p_min, int64_t p_max,
                             const bf16x8 (*qf)[D / 16], float c, RowState<D>& st,
                             const TileSmem<D>& sm) {
    if (k_lo >= k_hi) return;
    typedef typename TileCopySel<D, KV>::T TC;
    KeyLoop<D, KV> L;
    L.kv = kv;
    L.k_lo = k_lo;
    L.k_hi = k_hi;
    L.ks2 = (int)(kv.ks * 2);  // below 2^25 (host check) for flat storage
    L.vs2 = (int)(kv.vs * 2);
    if constexpr (std::is_same<KV, KVRing>::value) {
        L.kco = ring_offsets<D>(kv.R);
        L.vco = L.kco;
    } else {
        L.kco = copy_offsets<D>(L.ks2);
        L.vco = copy_offsets<D>(L.vs2);
    }
    interior_tiles<D>(L, causal, window, p_min, p_max);
    const int n = (k_hi - k_lo + kBN - 1) / kBN;
    L.n = n;
    LaneBounds lb[kNT];
#pragma unroll
    for (int nt = 0; nt < kNT; ++nt) lb[nt] = lane_bounds(k_lo, k_hi, causal, window, p_lane[nt]);
    const bool g1 = __builtin_amdgcn_readfirstlane(threadIdx.x / kWave) >= kWaves / 2;

    TileScores S;
    TileP pk;
    {
        const TC k0c = k_copy<D>(L, 0, sm.k[0]), k1c = k_copy<D>(L, 1, sm.k[1]);
        const TC v0c = v_copy<D>(L, 0, sm.v[0]);
#pragma unroll
        for (int i = 0; i < TC::N; ++i) {
            k0c.issue(i);
            k1c.issue(i);
            v0c.issue(i);
        }
    }
    TC ck = k_copy<D>(L, 2, sm.k[2]), cv = v_copy<D>(L, 1, sm.v[1]);
    tile_barrier();
    if (g1) phase_barrier();  // group 1 runs one phase behind
    // M(0): scores of tile 0, copies of K(2) and V(1)
    qk_tile<D>(sm.k[0], qf, S, ck, cv);
    pin_m_outputs<D>(S, st, true, false);
    copy_wait_barrier<2 * TC::N>();
    v_phase<D, true, false, KV, false, RS>(L, 0, c, lb, S, pk, st);  // tile 0 sets the references
    if (PRE) set_reference<D>(st);
    ck = k_copy<D>(L, 3, sm.k[0]);
    cv = v_copy<D>(L, 2, sm.v[2]);
    phase_barrier();
    int k = 1;
    for (; k + 2 < n; k += 3) {
        // k = 1 mod 3: K(k) in stage 1, V(k-1) in stage 0; copies of K(k+2) -> 0,
        // V(k+1) -> 2 (ck, cv); the next step's go to K stage 1, V stage 0
        pp_step<D, EXACT, PRE, KV, false, RS>(L, k, qf, c, lb, S, pk, st, sm.k[1], sm.v[0], ck, cv,
                                             sm.k[1], sm.v[0]);
        pp_step<D, EXACT, PRE, KV, false, RS>(L, k + 1, qf, c, lb, S, pk, st, sm.k[2], sm.v[1], ck,
                                             cv, sm.k[2], sm.v[1]);
        pp_step<D, EXACT, PRE, KV, kRefresh<D>, RS>(L, k + 2, qf, c, lb, S, pk, st, sm.k[0],
                                                   sm.v[2], ck, cv, sm.k[0], sm.v[2]);
    }
    if (k < n) {
        pp_step<D, EXACT, PRE, KV, false, RS>(L, k, qf, c, lb, S, pk, st, sm.k[1], sm.v[0], ck, cv,
                                             sm.k[1], sm.v[0]);
        ++k;
    }
    if (k < n) {
        pp_step<D, EXACT, PRE, KV, false, RS>(L, k, qf, c, lb, S, pk, st, sm.k[2], sm.v[1], ck, cv,
                                             sm.k[2], sm.v[1]);
        ++k;
    }
    // M(n): PV of tile n-1, whose V sits in stage (n-1) % 3; then no copy
    // is left in flight
    const int sv = (n - 1) % 3;
    if (sv == 0)
        pv_tile<D>(sm.v[0], pk, st, NoCopy{});
    else if (sv == 1)
        pv_tile<D>(sm.v[1], pk, st, NoCopy{});
    else
        pv_tile<D>(sm.v[2], pk, st, NoCopy{});
    copy_wait_barrier<0>();
    if (!g1) phase_barrier();  // matches group 1's extra barrier
}

// Q fragments of one row, zeros for rows that do not exist.  cq is the
// softmax scale times log2 e, sign included.  PS: Q times cq, rounded to
// bf16, so that the scores come out of the MFMAs in log2 units and the
// softmax takes c = 1.  Otherwise only the sign of cq is folded into Q
// (exact) and the softmax multiplies by c = |cq|.
template <int D, bool PS>
__device__ inline void load_q(bf16x8* qf, const u16* qrow, bool valid, float cq) {
    const int hh = (threadIdx.x & (kWave - 1)) >> 5;
#pragma unroll
    for (int kk = 0; kk < D / 16; ++kk) {
        const uint4 u = valid ? ld16(qrow + 16 * kk + 8 * hh) : make_uint4(0, 0, 0, 0);
        uint32_t w[4] = {u.x, u.y, u.z, u.w};
        if (PS) {
#pragma unroll
            for (int j = 0; j < 4; ++j)  // bf16 pair: element 0 in the low half
                w[j] = pack_bf16x2(__uint_as_float(w[j] << 16) * cq,
                                   __uint_as_float(w[j] & 0xffff0000u) * cq);
        }
        qf[kk] = __builtin_bit_cast(bf16x8, make_uint4(w[0], w[1], w[2], w[3]));
    }
    // exact Q: only a negative scale changes it (its sign, in a uniform
    // branch), so with a positive scale nothing waits for the loads here
    if (!PS && cq < 0.f) {
#pragma unroll
        for (int kk = 0; kk < D / 16; ++kk) {
            uint4 u = __builtin_bit_cast(uint4, qf[kk]);
            u.x ^= 0x80008000u;
            u.y ^= 0x80008000u;
            u.z ^= 0x80008000u;
            u.w ^= 0x80008000u;
            qf[kk] = __builtin_bit_cast(bf16x8, u);
        }
    }
}

typedef _Float16 f16x2 __attribute__((ext_vector_type(2)));
typedef unsigned u32x4 __attribute__((ext_vector_type(4)));

__device__ inline uint32_t pack_f16x2(float a, float b) {
    f32x2 v = {a, b};
    return __builtin_bit_cast(uint32_t, __builtin_convertvector(v, f16x2));
}

// Row stores through LDS.  The output accumulator leaves lane l of a wave
// with row l % 32 and the two half-waves with alternate groups of 4 values,
// so a direct store would write 16 bytes of each of 32 rows per
// instruction.  Instead the wave writes its rows, packed to 16 bits, into a
// private LDS tile (32 rows x D; the 16-byte chunk c of row r sits at chunk
// c ^ (r mod D/8), so that neither the writes nor the reads conflict on the
// banks), reads them back with D/8 consecutive lanes per row, and stores
// whole rows in 16-byte pieces (non-temporal for the fp16 split partials,
// which only the merge reads: measured 0.5-1 % faster on calls with
// splits).  rowp: this lane's row address, null when the row is not written
// (the same in both half-waves).  The tile must not be read or written by
// another wave meanwhile.
template <int D, bool F16>
__device__ inline void store_rows(const f32x16* o, float sc, u16* rowp, u16* tile) {
    constexpr int NC = D / 8, RPI = kWave / NC;  // chunks per row, rows per read
    const int lane = threadIdx.x & (kWave - 1), r = lane & 31, hh = lane >> 5;
#pragma unroll
    for (int dt = 0; dt < D / 32; ++dt)
#pragma unroll
        for (int a = 0; a < 4; ++a) {
            const int cc = 4 * dt + a;  // values 32dt + 8a + 4hh .. +3: chunk cc, half hh
            const float x0 = o[dt][4 * a] * sc, x1 = o[dt][4 * a + 1] * sc;
            const float x2 = o[dt][4 * a + 2] * sc, x3 = o[dt][4 * a + 3] * sc;
            const uint2 w = F16 ? make_uint2(pack_f16x2(x0, x1), pack_f16x2(x2, x3))
                                : make_uint2(pack_bf16x2(x0, x1), pack_bf16x2(x2, x3));
            *reinterpret_cast<uint2*>(tile + r * D + 8 * (cc ^ (r & (NC - 1))) + 4 * hh) = w;
        }
    // the reads below see the other lanes' writes (LDS keeps a wave's order)
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
    const uint64_t rp = (uint64_t)rowp;
    const int c = lane % NC;
#pragma unroll
    for (int j = 0; j < 32 / RPI; ++j) {
        const int R = j * RPI + lane / NC;
        const uint4 x = *reinterpret_cast<const uint4*>(tile + R * D + 8 * (c ^ (R & (NC - 1))));
        const uint32_t lo = (uint32_t)__builtin_amdgcn_ds_bpermute(R << 2, (int)(uint32_t)rp);
        const uint32_t hi =
            (uint32_t)__builtin_amdgcn_ds_bpermute(R << 2, (int)(uint32_t)(rp >> 32));
        u16* q = reinterpret_cast<u16*>(((uint64_t)hi << 32) | lo);
        if (q) {
            if (F16) {  // split partials: read once, by the merge
                const u32x4 xv = {x.x, x.y, x.z, x.w};
                __builtin_nontemporal_store(xv, reinterpret_cast<u32x4*>(q + 8 * c));
            } else {
                *reinterpret_cast<uint4*>(q + 8 * c) = x;
            }
        }
    }
}

// Final normalisation and bf16 store of one row: o / l, 0 when l == 0.
template <int D>
__device__ inline void store_out(const f32x16* o, float lpart, u16* orow, bool valid, u16* tile) {
    const float l = sum_across_halves(lpart);
    const float inv = l > 0.f ? 1.f / l : 0.f;
    store_rows<D, false>(o, inv, valid ? orow : nullptr, tile);
}

// Split partial of one row (prefill and varlen), at half the bytes of fp32:
// the accumulator divided by its sum (a convex combination of V rows) and by
// 2^e, with e the exponent of the row's largest |value| (clamped to
// [-100, 127]), so every element lies in [-1, 1]; rounded to fp16, where the
// rounding moves an element by at most 2^-12 of 2^e, i.e. 2^-11 of the row's
// largest value.  The record pml holds (m c or -inf when nothing was
// visible, l, l 2^e, 0) in fp32: the merge weighs the fp16 values by l 2^e.

template <int D>
__device__ inline void store_partial(const f32x16* o, float m, float lpart, float c, u16* po,
                                       float* pml, bool valid, u16* tile) {
    const int hh = (threadIdx.x & (kWave - 1)) >> 5;
    const float l = sum_across_halves(lpart);
    const float inv = l > 0.f ? 1.f / l : 0.f;
    float mx = 0.f;
#pragma unroll
    for (int dt = 0; dt < D / 32; ++dt)
#pragma unroll
        for (int r = 0; r < 16; ++r) mx = __builtin_fmaxf(mx, __builtin_fabsf(o[dt][r]));
    mx = max_across_halves(mx) * inv;
    int e = 0;
    (void)frexpf(mx, &e);  // mx < 2^e (e = 0 for mx = 0)
    e = e < -100 ? -100 : (e > 127 ? 127 : e);
    const float sc = ldexpf(inv, -e);
    store_rows<D, true>(o, sc, valid ? po : nullptr, tile);
    if (!valid) return;
    if (hh == 0)
        *reinterpret_cast<float4*>(pml) =
            make_float4(l > 0.f ? (m == -INFINITY ? 0.f : m * c) : -INFINITY, l, ldexpf(l, e), 0.f);
}

template <int D>
__device__ inline void init_state(RowState<D>& st) {
#pragma unroll
    for (int nt = 0; nt < kNT; ++nt) {
#pragma unroll
        for (int dt = 0; dt < D / 32; ++dt) st.o[nt][dt] = f32x16{};
        st.m[nt] = -INFINITY;
        st.l[nt] = 0.f;
        st.mneg[nt] = f32x16{};
    }
}

// Key range [lo, hi) of split `split` out of `nsplit` over [lo_all, hi_all).
__device__ inline void split_range(int lo_all, int hi_all, int split, int nsplit, int* lo, int* hi) {
    int span = hi_all - lo_all;
    int chunk = (span + nsplit - 1) / nsplit;
    chunk = (chunk + kBN - 1) / kBN * kBN;
    int a = lo_all + split * chunk;
    int b = a + chunk;
    *lo = a < hi_all ? a : hi_all;
    *hi = b < hi_all ? b : hi_all;
}

// Attend the keys [k_lo, k_hi) for the rows of the workgroup.  The first
// pass takes the exact maximum of the first tile as each row's reference
// and keeps it: later tiles need neither maxima nor rescales (softmax does
// not depend on the reference).  That is exact as long as no P overflows
// and the sum of a row that sees keys does not underflow, so every row
// checks that its sum lies in [2^-64, 2^64] (which bounds each P of the
// row); if any row of the workgroup fails, the workgroup redoes the range
// with the exact running-maximum pass.
//   PS: Q carries the scale (load_q<D, true>) and c = 1; the fixed-reference
//   pass then starts its score MFMAs from the negated references
//   (set_reference) and takes 2^s directly.
template <int D, bool PS, class KV>
__device__ bool attend(const KV& kv, int k_lo, int k_hi, int causal, int window,
                       const int64_t* p_lane, int64_t p_min, int64_t p_max,
                       const bf16x8 (*qf)[D / 16], float c, RowState<D>& st,
                       const TileSmem<D>& sm) {
    if (threadIdx.x == 0) *sm.rerun = 0;
    attend_range<D, false, PS, KV, !PS>(kv, k_lo, k_hi, causal, window, p_lane, p_min, p_max, qf, c, st,
                               sm);
    bool bad = false;
#pragma unroll
    for (int nt = 0; nt < kNT; ++nt) {
        const float l = sum_across_halves(st.l[nt]);
        const bool sees = lane_bounds(k_lo, k_hi, causal, window, p_lane[nt]).lo < k_hi;
        bad |= sees && !(l >= 0x1p-64f && l <= 0x1p64f);
    }
    if (__any(bad) && (threadIdx.x & (kWave - 1)) == 0) *sm.rerun = 1;
    __syncthreads();
    if (!*sm.rerun) return false;
    init_state<D>(st);
    attend_range<D, true, false, KV, true>(kv, k_lo, k_hi, causal, window, p_lane, p_min, p_max, qf, c, st,
                                 sm);
    return true;
}

// ---------------------------------------------------------------- prefill

// Largest magnitude of a query position read from the device (larger ones
// are clamped and flagged).
constexpr int64_t kBoundPos = (int64_t)1 << 62;

// Shader-clock sampling for the timing aid.  Thread 0 of each workgroup reads
// the shader cycle counter (s_memtime) and the constant 100 MHz reference
// counter (s_memrealtime) when it starts and when it is done, and adds both
// lifetimes to the sums of its XCD: clk[2x] shader cycles, clk[2x+1]
// reference ticks.  The ratio is the average shader clock while the
// workgroups ran.  clk[16] counts the workgroups that added to the sums and
// clk[17] those among them whose fixed-reference pass had to be redone with
// the exact running maximum.  clk is null unless timing is on.
__device__ unsigned long long g_clock[18];

struct ClockMark {
    unsigned long long cyc, ref;
};

__device__ inline ClockMark clock_mark(const unsigned long long* clk) {
    ClockMark m{0, 0};
    if (clk) {  // uniform: the counters are read into scalar registers
        m.cyc = __builtin_amdgcn_s_memtime();
        m.ref = __builtin_amdgcn_s_memrealtime();
    }
    return m;
}

__device__ inline void clock_add(unsigned long long* clk, ClockMark m, bool redone = false) {
    if (clk) {
        const unsigned long long cyc = __builtin_amdgcn_s_memtime();
        const unsigned long long ref = __builtin_amdgcn_s_memrealtime();
        unsigned xcc;
        asm volatile("s_getreg_b32 %0, hwreg(HW_REG_XCC_ID)" : "=s"(xcc));
        xcc &= 7;
        if (threadIdx.x == 0) {  // vector atomics from one lane
            atomicAdd(clk + 2 * xcc, cyc - m.cyc);
            atomicAdd(clk + 2 * xcc + 1, ref - m.ref);
            atomicAdd(clk + 16, 1ull);
            if (redone) atomicAdd(clk + 17, 1ull);
        }
    }
}

struct PrefillArgs {
    const u16* q;
    const u16* k;
    const u16* v;
    u16* out;
    u16* part_o;     // [nsplit][B][Hq][Lq][D] fp16 bits (store_partial)
    float* part_ml;  // [nsplit][B][Hq][Lq][4]
    int B, Hq, Hkv, Lq, Lkv, window, nsplit;
    int n_inner;  // q blocks x head chunks
    float c;  // |scale| * log2(e)
    int negate;
    int64_t q_pos0;
    int64_t qs[4], ks[4], vs[4], os[4];
    unsigned long long* clk;  // timing aid: per-XCD clock sums, or null
    const int64_t* bounds;    // device (q_pos0, kv_len) replacing q_pos0 and Lkv, or null
    int32_t* err;             // with bounds: the bound flags, written by workgroup 0
};

// Workgroups are dispatched to the 8 XCDs round-robin by linear id.  Map
// linear id L to work item w so that each XCD receives a contiguous range of
// work items (a bijection on [0, N)); consecutive work items share their
// K/V range, so each XCD's L2 streams its own slice of K/V.
__device__ inline int xcd_remap(int L, int N) {
    constexpr int X = 8;
    const int per = N / X, rem = N % X;
    const int x = L % X, i = L / X;
    return x < rem ? x * (per + 1) + i : rem * (per + 1) + (x - rem) * per + i;
}

#define DECLARE_TILE_SMEM(D)                                                              \
    __shared__ __attribute__((aligned(1024))) u16 sk0[kBN * (D)];                        \
    __shared__ __attribute__((aligned(1024))) u16 sv0[kBN * (D)];                        \
    __shared__ __attribute__((aligned(1024))) u16 sk1[kBN * (D)];                        \
    __shared__ __attribute__((aligned(1024))) u16 sv1[kBN * (D)];                        \
    __shared__ __attribute__((aligned(1024))) u16 sk2[kBN * (D)];                        \
    __shared__ __attribute__((aligned(1024))) u16 sv2[kBN * (D)];                        \
    __shared__ int rerun_flag;                                                           \
    const TileSmem<D> sm{{sk0, sk1, sk2}, {sv0, sv1, sv2}, &rerun_flag}

// PS: Q carries the scale (chosen by the host for |scale| <= 1/sqrt(D)).
template <int D, bool PS>
__global__ __launch_bounds__(kThreads) void prefill_kernel(PrefillArgs a) {
    DECLARE_TILE_SMEM(D);
    const ClockMark cm = clock_mark(a.clk);

    const int g = a.Hq / a.Hkv;
    const RowMap rm = row_map(g);
    // work item: outer (b, hk, split), inner (q block, head chunk)
    const int w = xcd_remap(blockIdx.x, gridDim.x);
    const int inner = w % a.n_inner, outer = w / a.n_inner;
    const int qb = inner / rm.hchunks, hc = inner % rm.hchunks;
    const int split = outer % a.nsplit, bh = outer / a.nsplit;
    const int b = bh / a.Hkv, hk = bh % a.Hkv;
    const int q0 = qb * rm.P;
    const int heads_here = min(rm.Gc, g - hc * rm.Gc);

    const int wave = threadIdx.x / kWave, lane = threadIdx.x & (kWave - 1);
    // the key bound and the first row's position: from the call, or read on
    // the device (Lkv is then the capacity: a larger bound is clamped to it)
    int64_t q_pos0 = a.q_pos0;
    int Lkv = a.Lkv;
    if (a.bounds) {
        const int64_t qp = a.bounds[0], kl = a.bounds[1];
        q_pos0 = qp < -kBoundPos ? -kBoundPos : (qp > kBoundPos ? kBoundPos : qp);
        Lkv = kl < 0 ? 0 : (kl > a.Lkv ? a.Lkv : (int)kl);
        if (blockIdx.x == 0 && threadIdx.x == 0)
            a.err[0] = (kl < 0 || kl > a.Lkv ? ATTN_BOUND_KV : 0) |
                       (qp != q_pos0 ? ATTN_BOUND_QPOS : 0);
    }
    const int64_t p_min = q_pos0 + q0;
    const int64_t p_max = q_pos0 + min(q0 + rm.P, a.Lq) - 1;

    // this lane's row in each of the wave's row tiles
    int hrow[kNT], irow[kNT];
    bool valid[kNT];
    int64_t p_lane[kNT];
    bf16x8 qf[kNT][D / 16];
#pragma unroll
    for (int nt = 0; nt < kNT; ++nt) {
        const int r = (wave * kNT + nt) * 32 + (lane & 31);
        const int hl = r / rm.P, pos = r % rm.P;
        irow[nt] = q0 + pos;
        hrow[nt] = hk * g + hc * rm.Gc + hl;
        valid[nt] = hl < heads_here && irow[nt] < a.Lq;
        p_lane[nt] = valid[nt] ? q_pos0 + irow[nt] : p_max;
        load_q<D, PS>(qf[nt],
                      a.q + b * a.qs[0] + (int64_t)hrow[nt] * a.qs[1] + (int64_t)irow[nt] * a.qs[2],
                      valid[nt], a.negate ? -a.c : a.c);
    }

    // visible keys of the whole workgroup, then this split's share
    int64_t lo64 = a.window > 0 ? p_min - a.window + 1 : 0;
    int64_t hi64 = p_max + 1 < Lkv ? p_max + 1 : Lkv;
    if (lo64 < 0) lo64 = 0;
    if (hi64 < lo64) hi64 = lo64;
    int k_lo, k_hi;
    split_range((int)lo64, (int)hi64, split, a.nsplit, &k_lo, &k_hi);

    RowState<D> st;
    init_state<D>(st);
    KVFlat kv{a.k + b * a.ks[0] + hk * a.ks[1], a.v + b * a.vs[0] + hk * a.vs[1], a.ks[2],
              a.vs[2]};
    const float c = PS ? 1.f : a.c;
    const bool redone = attend<D, PS>(kv, k_lo, k_hi, 1, a.window, p_lane, p_min, p_max, qf, c, st, sm);

    static_assert(kNT == 1, "one row tile per wave");
    u16* const tile = row_tile<D>(sm, __builtin_amdgcn_readfirstlane(wave));
    __syncthreads();  // every wave is done with the stages
    if (a.nsplit == 1) {
        store_out<D>(st.o[0], st.l[0],
                     a.out + b * a.os[0] + (int64_t)hrow[0] * a.os[1] + (int64_t)irow[0] * a.os[2],
                     valid[0], tile);
    } else {
        const int64_t row = (((int64_t)split * a.B + b) * a.Hq + hrow[0]) * a.Lq + irow[0];
        store_partial<D>(st.o[0], st.m[0], st.l[0], c, a.part_o + row * D, a.part_ml + row * 4,
                         valid[0], tile);
    }
    clock_add(a.clk, cm, redone);
}

// ---------------------------------------------------------------- D = 256
//
// Head dimension 256 does not fit the ping-pong kernel: a wave's 32 rows
// hold 128 accumulator and 64 query-fragment registers, so only one wave
// fits per SIMD.  The workgroup is four waves (128 rows, one wave per SIMD)
// over 64-key K and V tiles double-buffered in LDS (4 x 32 KB): while the
// waves compute tile t, the copies of tile t+1 are in flight.  The softmax
// is the fixed-reference pass with an exact rerun, as in the prefill kernel.

constexpr int kWaves256 = 4;
constexpr int kBM256 = kWaves256 * 32;

typedef TileCopyFlat<256, kWaves256> Copy256;
typedef CopyOffsets<256, kWaves256> Offs256;

// This wave's share of the copy of keys [k0, k0 + 64) of one tensor into an
// LDS tile (zeros for rows at or past k_hi).
__device__ inline void copy_tile256(const u16* base, int64_t rs, const Offs256& co, int k0,
                                    int k_hi, u16* dst) {
    const Copy256 cp(KVFlat{}, base, rs, (int)(rs * 2), co, k0 < k_hi ? k0 : k_hi, k_hi, dst);
#pragma unroll
    for (int i = 0; i < Copy256::N; ++i) cp.issue(i);
}

// One key tile of the D = 256 loop.  The wave waits for its copies of this
// tile, and the workgroup barrier makes every wave's copies visible and
// tells that every wave is done with the previous tile's stages (Kn, Vn);
// the copies of the next tile into them are spread between the MFMAs of the
// scores, then mask, softmax, PV.  (Issued before the barrier instead, the
// copies made the compiler wait for the K copy before the first K read.)
// The softmax is that of the prefill kernel: EXACT, against each row's
// running maximum; otherwise tile 0 sets a fixed reference and later tiles
// neither take maxima nor rescale (the caller checks the sums).
template <bool EXACT, bool FIRST, bool PS>
__device__ inline void tile256(const u16* kb, const u16* vb, int64_t krs, int64_t vrs,
                               const Offs256& kco, const Offs256& vco, int t,
                               int n, int k_lo, int k_hi, int t_in0, int t_in1,
                               const bf16x8 (*qf)[16], const LaneBounds* lb, float c,
                               RowState<256>& st, const u16* Kc, const u16* Vc, u16* Kn, u16* Vn) {
    constexpr int D = 256;
    __builtin_amdgcn_s_waitcnt(0x0F70);  // vmcnt(0)
    __builtin_amdgcn_s_barrier();
    // past the range: zeros into stages nobody reads, no memory touched
    const int k1 = t + 1 < n ? k_lo + (t + 1) * kBN : k_hi;
    const Copy256 ck(KVFlat{}, kb, krs, (int)(krs * 2), kco, k1, k_hi, Kn);
    const Copy256 cv(KVFlat{}, vb, vrs, (int)(vrs * 2), vco, k1, k_hi, Vn);
    constexpr bool PRE = PS && !EXACT && !FIRST;  // scores come out as s - m
    TileScores S;
    qk_tile<D, Copy256, Copy256, PRE>(Kc, qf, S, ck, cv, st.mneg);
    if (t < t_in0 || t >= t_in1) mask_tile(S, k_lo + t * kBN, lb);
    float lsum[kNT];
    if (EXACT || FIRST) {
        float alpha[kNT];
        update_max(S, c, st.m, alpha);
        if (!FIRST) rescale<D>(alpha, st);  // tile 0: O and l are still zero
        if (PS && FIRST && !EXACT) set_reference<D>(st);
    }
    TileP pk;
    softmax_tile<PRE, !PS>(S, c, st.m, pk, lsum);
    st.l[0] += lsum[0];
    pv_tile<D>(Vc, pk, st, NoCopy{});
}

// PS: as prefill_kernel.
template <bool PS>
__global__ __launch_bounds__(kWaves256 * kWave, 1) void prefill256_kernel(PrefillArgs a) {
    constexpr int D = 256;
    __shared__ __attribute__((aligned(1024))) u16 sk0[kBN * D];
    __shared__ __attribute__((aligned(1024))) u16 sv0[kBN * D];
    __shared__ __attribute__((aligned(1024))) u16 sk1[kBN * D];
    __shared__ __attribute__((aligned(1024))) u16 sv1[kBN * D];
    const ClockMark cm = clock_mark(a.clk);

    const int g = a.Hq / a.Hkv;
    const RowMap rm = row_map(g, kBM256);
    const int w = xcd_remap(blockIdx.x, gridDim.x);
    const int inner = w % a.n_inner, outer = w / a.n_inner;
    const int qb = inner / rm.hchunks, hc = inner % rm.hchunks;
    const int split = outer % a.nsplit, bh = outer / a.nsplit;
    const int b = bh / a.Hkv, hk = bh % a.Hkv;
    const int q0 = qb * rm.P;
    const int heads_here = min(rm.Gc, g - hc * rm.Gc);

    int64_t q_pos0 = a.q_pos0;
    int Lkv = a.Lkv;
    if (a.bounds) {
        const int64_t qp = a.bounds[0], kl = a.bounds[1];
        q_pos0 = qp < -kBoundPos ? -kBoundPos : (qp > kBoundPos ? kBoundPos : qp);
        Lkv = kl < 0 ? 0 : (kl > a.Lkv ? a.Lkv : (int)kl);
        if (blockIdx.x == 0 && threadIdx.x == 0)
            a.err[0] = (kl < 0 || kl > a.Lkv ? ATTN_BOUND_KV : 0) |
                       (qp != q_pos0 ? ATTN_BOUND_QPOS : 0);
    }
    const int64_t p_min = q_pos0 + q0;
    const int64_t p_max = q_pos0 + min(q0 + rm.P, a.Lq) - 1;

    const int wave = threadIdx.x / kWave, lane = threadIdx.x & (kWave - 1);
    const int r = wave * 32 + (lane & 31);
    const int hl = r / rm.P, pos = r % rm.P;
    const int irow = q0 + pos, hrow = hk * g + hc * rm.Gc + hl;
    const bool valid = hl < heads_here && irow < a.Lq;
    const int64_t p_lane = valid ? q_pos0 + irow : p_max;
    bf16x8 qf[1][D / 16];
    load_q<D, PS>(qf[0], a.q + b * a.qs[0] + (int64_t)hrow * a.qs[1] + (int64_t)irow * a.qs[2],
                  valid, a.negate ? -a.c : a.c);
    const float c = PS ? 1.f : a.c;

    int64_t lo64 = a.window > 0 ? p_min - a.window + 1 : 0;
    int64_t hi64 = p_max + 1 < Lkv ? p_max + 1 : Lkv;
    if (lo64 < 0) lo64 = 0;
    if (hi64 < lo64) hi64 = lo64;
    int k_lo, k_hi;
    split_range((int)lo64, (int)hi64, split, a.nsplit, &k_lo, &k_hi);

    RowState<D> st;
    init_state<D>(st);
    bool redone = false;
    if (k_lo < k_hi) {
        const int n = (k_hi - k_lo + kBN - 1) / kBN;
        // tiles t_in0 <= t < t_in1 need no mask (as interior_tiles)
        int64_t t1 = (k_hi - k_lo) / kBN;
        {
            const int64_t cc = p_min - k_lo - (kBN - 1);
            const int64_t tc = cc < 0 ? 0 : cc / kBN + 1;
            if (tc < t1) t1 = tc;
        }
        int64_t t0 = 0;
        if (a.window > 0) {
            const int64_t ww = p_max - a.window - k_lo;
            t0 = ww < 0 ? 0 : ww / kBN + 1;
        }
        if (t1 > n) t1 = n;
        if (t0 > t1) t0 = t1;
        const LaneBounds lb = lane_bounds(k_lo, k_hi, 1, a.window, p_lane);
        const u16* kb = a.k + b * a.ks[0] + hk * a.ks[1];
        const u16* vb = a.v + b * a.vs[0] + hk * a.vs[1];
        const Offs256 kco = copy_offsets<D, kWaves256>((int)(a.ks[2] * 2));
        const Offs256 vco = copy_offsets<D, kWaves256>((int)(a.vs[2] * 2));
        // the fixed-reference pass, then the exact one if a row's sum left
        // [2^-64, 2^64] (as the prefill kernel)
        __shared__ int rerun;
        if (threadIdx.x == 0) rerun = 0;
        copy_tile256(kb, a.ks[2], kco, k_lo, k_hi, sk0);
        copy_tile256(vb, a.vs[2], vco, k_lo, k_hi, sv0);
        tile256<false, true, PS>(kb, vb, a.ks[2], a.vs[2], kco, vco, 0, n, k_lo, k_hi, (int)t0,
                             (int)t1, qf, &lb, c, st, sk0, sv0, sk1, sv1);
        for (int t = 1; t < n; t += 2) {
            tile256<false, false, PS>(kb, vb, a.ks[2], a.vs[2], kco, vco, t, n, k_lo, k_hi, (int)t0, (int)t1,
                           qf, &lb, c, st, sk1, sv1, sk0, sv0);
            if (t + 1 < n)
                tile256<false, false, PS>(kb, vb, a.ks[2], a.vs[2], kco, vco, t + 1, n, k_lo, k_hi, (int)t0,
                               (int)t1, qf, &lb, c, st, sk0, sv0, sk1, sv1);
        }
        __builtin_amdgcn_s_waitcnt(0x0F70);  // the last tile's (empty) copies
        const float lrow = sum_across_halves(st.l[0]);
        const bool bad = lb.lo < k_hi && !(lrow >= 0x1p-64f && lrow <= 0x1p64f);
        if (__any(bad) && lane == 0) rerun = 1;
        __syncthreads();
        redone = rerun != 0;
        if (redone) {
            init_state<D>(st);
            copy_tile256(kb, a.ks[2], kco, k_lo, k_hi, sk0);
            copy_tile256(vb, a.vs[2], vco, k_lo, k_hi, sv0);
            for (int t = 0; t < n; t += 2) {
                tile256<true, false, PS>(kb, vb, a.ks[2], a.vs[2], kco, vco, t, n, k_lo, k_hi, (int)t0,
                              (int)t1, qf, &lb, c, st, sk0, sv0, sk1, sv1);
                if (t + 1 < n)
                    tile256<true, false, PS>(kb, vb, a.ks[2], a.vs[2], kco, vco, t + 1, n, k_lo, k_hi,
                                  (int)t0, (int)t1, qf, &lb, c, st, sk1, sv1, sk0, sv0);
            }
            __builtin_amdgcn_s_waitcnt(0x0F70);
        }
    }

    // row-store tiles: two waves per stage; every wave is done with them
    const int wv = __builtin_amdgcn_readfirstlane(threadIdx.x / kWave);
    u16* const tile = (wv < 2 ? sk0 : sv0) + (wv & 1) * 32 * D;
    __syncthreads();
    if (a.nsplit == 1) {
        store_out<D>(st.o[0], st.l[0],
                     a.out + b * a.os[0] + (int64_t)hrow * a.os[1] + (int64_t)irow * a.os[2],
                     valid, tile);
    } else {
        const int64_t row =
            (((int64_t)split * a.B + b) * a.Hq + hrow) * a.Lq + irow;
        store_partial<D>(st.o[0], st.m[0], st.l[0], c, a.part_o + row * D, a.part_ml + row * 4,
                           valid, tile);
    }
    clock_add(a.clk, cm, redone);
}

// Merge the split partials (store_partial) of one row: M = max m_s, w_s =
// 2^(m_s - M); split s adds w_s l_s 2^e_s times its fp16 values to the
// numerator and w_s l_s to the denominator; o = numerator / denominator (0
// when it is 0).  This thread merges the 8 values [d0, d0 + 8), one 16-byte
// load per split.  The splits are read in groups of G whose loads are all in
// flight together (indices past nsplit are clamped and weighted 0); groups
// merge by the same rule.
template <int D, int G>
__device__ inline void combine_row(const u16* po, const float* pml, int64_t split_stride_o,
                                     int64_t split_stride_ml, int nsplit, int d0, u16* orow) {
    constexpr int W = 8;
    float M = -INFINITY, L = 0.f;
    float acc[W];
#pragma unroll
    for (int i = 0; i < W; ++i) acc[i] = 0.f;
    for (int s0 = 0; s0 < nsplit; s0 += G) {
        float4 r[G];
        uint4 x[G];
#pragma unroll
        for (int j = 0; j < G; ++j) {
            const int sj = min(s0 + j, nsplit - 1);
            r[j] = *reinterpret_cast<const float4*>(pml + sj * split_stride_ml);
            x[j] = *reinterpret_cast<const uint4*>(po + sj * split_stride_o + d0);
        }
        float Mg = M;
#pragma unroll
        for (int j = 0; j < G; ++j)
            if (s0 + j < nsplit) Mg = __builtin_fmaxf(Mg, r[j].x);
        if (Mg == -INFINITY) continue;  // nothing visible so far
        const float rs = M == -INFINITY ? 0.f : __builtin_amdgcn_exp2f(M - Mg);
        L *= rs;
#pragma unroll
        for (int i = 0; i < W; ++i) acc[i] *= rs;
#pragma unroll
        for (int j = 0; j < G; ++j) {
            const float w = (s0 + j < nsplit && r[j].x != -INFINITY)
                                ? __builtin_amdgcn_exp2f(r[j].x - Mg) : 0.f;
            const float wz = w * r[j].z;
            L += w * r[j].y;
            const uint32_t h[4] = {x[j].x, x[j].y, x[j].z, x[j].w};
#pragma unroll
            for (int k = 0; k < W / 2; ++k) {
                const f16x2 p2 = __builtin_bit_cast(f16x2, h[k]);
                acc[2 * k] += wz * (float)p2[0];
                acc[2 * k + 1] += wz * (float)p2[1];
            }
        }
        M = Mg;
    }
    const float inv = L > 0.f ? 1.f / L : 0.f;
    *reinterpret_cast<uint4*>(orow + d0) =
        make_uint4(pack_bf16x2(acc[0] * inv, acc[1] * inv), pack_bf16x2(acc[2] * inv, acc[3] * inv),
                   pack_bf16x2(acc[4] * inv, acc[5] * inv), pack_bf16x2(acc[6] * inv, acc[7] * inv));
}

template <int D>
__global__ __launch_bounds__(256) void prefill_combine_kernel(PrefillArgs a) {
    constexpr int TPR = D / 8;  // threads per row, 8 dims each (one 16-byte load per split)
    int64_t rows = (int64_t)a.B * a.Hq * a.Lq;
    int64_t row = (int64_t)blockIdx.x * (256 / TPR) + threadIdx.x / TPR;
    if (row >= rows) return;
    int d0 = (threadIdx.x % TPR) * 8;
    int i = (int)(row % a.Lq);
    int h = (int)((row / a.Lq) % a.Hq);
    int b = (int)(row / ((int64_t)a.Lq * a.Hq));
    u16* orow = a.out + b * a.os[0] + (int64_t)h * a.os[1] + (int64_t)i * a.os[2];
    // loads of every split in flight at once, in the narrowest group that
    // holds them (no clamped duplicates)
    if (a.nsplit <= 4)
        combine_row<D, 4>(a.part_o + row * D, a.part_ml + row * 4, rows * D, rows * 4,
                             a.nsplit, d0, orow);
    else
        combine_row<D, 8>(a.part_o + row * D, a.part_ml + row * 4, rows * D, rows * 4,
                             a.nsplit, d0, orow);
}

// ---------------------------------------------------------------- varlen

struct VarlenArgs {
    const u16* q;
    const u16* k;
    const u16* v;
    u16* out;
    const int32_t* seq_info;
    const int32_t* seg_attr;
    int32_t* err;    // one word per finish workgroup
    u16* part_o;     // split partials per packed row: [T][Hq][nsplit][D], fp16 bits
    float* part_ml;  // [T][Hq][nsplit][4] (store_partial records)
    int S, T, Hq, Hkv, rows, cols, causal, window, ring_rows;
    int nsplit;      // most key splits of a q-block
    int split_keys;  // target keys per split (the finest, when adaptive)
    int adaptive;    // choose the split per table (choose_split_wave); at most 64 segments
    int gx;          // workgroups of the attention launch
    float c;
    int negate;
    int64_t qs[3], ks[4], vs[4], os[3];
    unsigned long long* clk;  // timing aid: per-XCD clock sums, or null
};

struct Segment {
    int q_start, q_len, col, kv_end;
    int causal, window, R;
    int flags;
};

// Decode and check segment s (the same rules as ATTN_SEG_* in attn.h).
__device__ inline Segment read_segment(const VarlenArgs& a, int s) {
    Segment g;
    g.q_start = a.seq_info[4 * s + 0];
    g.q_len = a.seq_info[4 * s + 1];
    g.col = a.seq_info[4 * s + 2];
    g.kv_end = a.seq_info[4 * s + 3];
    int ring_rows;
    if (a.seg_attr) {
        g.causal = a.seg_attr[3 * s + 0];
        g.window = a.seg_attr[3 * s + 1];
        ring_rows = a.seg_attr[3 * s + 2];
    } else {
        g.causal = a.causal;
        g.window = a.window;
        ring_rows = a.ring_rows;
    }
    int f = 0;
    if (g.q_start < 0 || g.q_len < 0 || (int64_t)g.q_start + g.q_len > a.T) f |= ATTN_SEG_QRANGE;
    if (g.col < 0 || g.col >= a.cols - 1) f |= ATTN_SEG_COL;
    if (ring_rows > a.rows) f |= ATTN_SEG_ATTR;
    bool ring = ring_rows > 0;
    g.R = ring ? ring_rows : a.rows;
    if (g.kv_end < 0 || (!ring && g.kv_end > a.rows)) f |= ATTN_SEG_KVEND;
    // a ring of R rows holds positions kv_end - R .. kv_end - 1 only; the
    // earliest key any query of the segment sees is its first query's
    if (ring && g.q_len > 0 && g.kv_end > 0) {
        int64_t first = g.window > 0 ? (int64_t)g.kv_end - g.q_len - g.window + 1 : 0;
        if (first < 0) first = 0;
        if ((int64_t)g.kv_end - first > g.R) f |= ATTN_SEG_SPAN;
    }
    g.flags = f;
    return g;
}

// Visible key range [lo, hi) of q-block qb (P positions) of segment g.
__device__ inline void block_range(const Segment& g, int qb, int P, int64_t* lo, int64_t* hi,
                                   int64_t* p_min, int64_t* p_max) {
    const int64_t base = (int64_t)g.kv_end - g.q_len;
    *p_min = base + (int64_t)qb * P;
    *p_max = base + min(qb * P + P, g.q_len) - 1;
    int64_t l = g.window > 0 ? *p_min - g.window + 1 : 0;
    int64_t h = g.kv_end;
    if (g.causal && *p_max + 1 < h) h = *p_max + 1;
    if (l < 0) l = 0;
    if (h < l) h = l;
    *lo = l;
    *hi = h;
}

// Work items of one segment: each of its nqb q-blocks, for every (kv head,
// head chunk) pair (hg of them), splits its visible keys into nsplit chunks
// of about split_keys keys.  cost = 64-key tiles of its largest item, the
// key by which items are ordered longest first.  The largest key range of a
// segment's q-blocks is its first or its last one's (the range size is
// monotone in the block index in every mode).
//
// A segment whose rows (q_len positions x the gq query heads of a kv head)
// fit one 32-row tile is planned as decode items instead: one per (kv head,
// split), its whole q_len in one block (see decode_item).  Their cost counts
// the 64-key tiles of one wave, plus one for the latency of the first.
struct SegPlan {
    int nqb, nsplit, cost, count;
    bool decode;
};

__device__ inline bool decode_rows(int gq, int q_len) { return gq * q_len <= 32; }

__device__ inline SegPlan seg_plan(const Segment& g, int P, int hg, int gq, int hkv, int split_keys,
                                   int nsplit_max) {
    SegPlan p{0, 1, 0, 0, false};
    if (g.flags || g.q_len <= 0) return p;
    p.decode = decode_rows(gq, g.q_len);
    const int Pb = p.decode ? g.q_len : P;  // positions per q-block
    p.nqb = (g.q_len + Pb - 1) / Pb;
    int64_t lo, hi, pmn, pmx, lo1, hi1;
    block_range(g, 0, Pb, &lo, &hi, &pmn, &pmx);
    block_range(g, p.nqb - 1, Pb, &lo1, &hi1, &pmn, &pmx);
    // a range lies inside [0, kv_end), kv_end < 2^31: 32-bit divisions
    const unsigned span = (unsigned)max(hi - lo, hi1 - lo1);
    const unsigned n = (span + (unsigned)split_keys - 1u) / (unsigned)split_keys;
    p.nsplit = n < 1u ? 1 : (n > (unsigned)nsplit_max ? nsplit_max : (int)n);
    const unsigned tiles = (span / (unsigned)p.nsplit + (span % (unsigned)p.nsplit != 0) + kBN - 1) / kBN;
    p.cost = (int)min(0x3fffffffu, p.decode ? (tiles + kWaves - 1) / kWaves + 1 : tiles);
    p.count = p.decode ? hkv * p.nsplit : p.nqb * hg * p.nsplit;
    return p;
}

// The work item of linear index L: items are ordered by their segment's
// cost, largest first (ties in table order), so the hardware dispatcher,
// which starts workgroups in index order on whichever compute unit frees up,
// schedules longest items first.  Each thread plans its own segments, then
// sums the item counts of the segments ordered before them; one thread finds
// the segment that holds L.  Returns false when L is past the last item.
__device__ bool pick_item(const VarlenArgs& a, int P, int hg, int gq, int L, int* seg_out,
                          int* j_out, Segment* sg_out) {
    constexpr int NT = kThreads;  // one segment per thread per pass
    __shared__ int sh_cost[NT], sh_count[NT];
    __shared__ int sh_seg, sh_j;
    __shared__ Segment sh_sg;
    if (threadIdx.x == 0) sh_seg = -1;
    for (int c0 = 0; c0 < a.S; c0 += NT) {
        const int s = c0 + threadIdx.x;
        const Segment xs = s < a.S ? read_segment(a, s) : Segment{};
        const SegPlan ps = s < a.S ? seg_plan(xs, P, hg, gq, a.Hkv, a.split_keys, a.nsplit)
                                   : SegPlan{0, 1, 0, 0, false};
        int64_t off = 0;
        for (int d0 = 0; d0 < a.S; d0 += NT) {
            const int s2 = d0 + threadIdx.x;
            SegPlan p2 = ps;
            if (d0 != c0)
                p2 = s2 < a.S ? seg_plan(read_segment(a, s2), P, hg, gq, a.Hkv, a.split_keys,
                                         a.nsplit)
                              : SegPlan{0, 1, 0, 0, false};
            __syncthreads();
            sh_cost[threadIdx.x] = p2.cost;
            sh_count[threadIdx.x] = p2.count;
            __syncthreads();
            const int n = min(NT, a.S - d0);
            for (int i = 0; i < n; ++i) {
                const int c2 = sh_cost[i];
                if (c2 > ps.cost || (c2 == ps.cost && d0 + i < s)) off += sh_count[i];
            }
        }
        if (s < a.S && ps.count > 0 && L >= off && L < off + ps.count) {
            sh_seg = s;
            sh_j = (int)(L - off);
            sh_sg = xs;  // the picked segment, so no thread reads it again
        }
    }
    __syncthreads();
    *seg_out = sh_seg;
    *j_out = sh_j;
    if (sh_seg >= 0) *sg_out = sh_sg;
    return sh_seg >= 0;
}

// Split size for this table, chosen by each wave on its own (lane i plans
// segment i): the finest of split_keys, x 1.5, x 1.5^2, ... whose items fit
// the launch, so that a table with many q-blocks takes longer splits and
// fewer items (one item per workgroup and no empty workgroups when its
// items fit one round), while one with few rows keeps fine splits.  At
// split_keys >= rows no range splits, and the launch (at least one
// workgroup per q-block slot) holds every item of a table whose segments
// do not overlap.  The same arithmetic on the same table gives every wave
// of the attention launch and of the finish pass the same choice.  Returns
// the split size and, in *plan, this lane's segment plan at that size.
__device__ inline int choose_split_wave(const VarlenArgs& a, const Segment& xs, bool has, int P,
                                        int hg, int gq, SegPlan* plan) {
    int sk = a.split_keys;
    for (;;) {
        const SegPlan p = has ? seg_plan(xs, P, hg, gq, a.Hkv, sk, a.nsplit)
                              : SegPlan{0, 1, 0, 0, false};
        int n = 0;  // the items of the table: a scalar sum over the segments' lanes
        for (int i = 0; i < a.S; ++i) n += __builtin_amdgcn_readlane(p.count, i);
        if (n <= a.gx || sk >= a.rows) {
            *plan = p;
            return sk;
        }
        sk += sk >> 1;
    }
}

// The same choice made by each wave on its own when the table has at most
// 64 segments: lane i plans segment i, and each lane sums the item counts of
// the segments ordered before its own from the other lanes' plans (readlane),
// so there is no LDS and no barrier, and one round of table loads.
__device__ bool pick_item_wave(const VarlenArgs& a, int P, int hg, int gq, int L, int* j_out,
                               Segment* sg_out, int* sk_out) {
    const int lane = threadIdx.x & (kWave - 1);
    const bool has = lane < a.S;
    const Segment xs = has ? read_segment(a, lane) : Segment{};
    SegPlan ps;
    int sk = a.split_keys;
    if (a.adaptive)
        sk = choose_split_wave(a, xs, has, P, hg, gq, &ps);
    else
        ps = has ? seg_plan(xs, P, hg, gq, a.Hkv, sk, a.nsplit) : SegPlan{0, 1, 0, 0, false};
    *sk_out = sk;
    int64_t off = 0;
    for (int i = 0; i < a.S; ++i) {
        const int c2 = __builtin_amdgcn_readlane(ps.cost, i);
        const int n2 = __builtin_amdgcn_readlane(ps.count, i);
        if (c2 > ps.cost || (c2 == ps.cost && i < lane)) off += n2;
    }
    const bool mine = has && ps.count > 0 && L >= off && L < off + ps.count;
    const uint64_t m = __ballot(mine);
    if (!m) return false;
    const int w = __builtin_ctzll(m);  // the item ranges are disjoint: one lane
    *j_out = __builtin_amdgcn_readlane((int)(L - off), w);
    sg_out->q_start = __builtin_amdgcn_readlane(xs.q_start, w);
    sg_out->q_len = __builtin_amdgcn_readlane(xs.q_len, w);
    sg_out->col = __builtin_amdgcn_readlane(xs.col, w);
    sg_out->kv_end = __builtin_amdgcn_readlane(xs.kv_end, w);
    sg_out->causal = __builtin_amdgcn_readlane(xs.causal, w);
    sg_out->window = __builtin_amdgcn_readlane(xs.window, w);
    sg_out->R = __builtin_amdgcn_readlane(xs.R, w);
    sg_out->flags = 0;
    return true;
}

// ---------------------------------------------------------------- decode items
//
// Few rows and many keys: such an item is bound by the K/V stream, so every
// wave streams its own key tiles instead of sharing one pipeline.  Wave w
// takes the 64-key tiles w, w + 8, ... of the split's range, each with the
// item's (at most 32) rows: K straight into the MFMA operand registers, V
// into the wave's own LDS tile (the transposing reads need it there), then
// the exact online softmax.  With one tile in flight per wave, a workgroup
// keeps eight tiles of loads outstanding.  The eight states then merge
// through LDS into one partial (or the output when the range is not split).

// K operand registers of one 64-key tile: lane l holds key k0 + 32t + l%32,
// d = 16kk + 8(l/32) .. +8 (the layout k_frag reads from LDS).  Keys at or
// past k_hi repeat key k_hi - 1 (their scores are masked).
template <int D>
__device__ inline void load_k_regs(bf16x8 (&kr)[2][D / 16], const KVRing& kv, int k0, int k_hi) {
    const int lane = threadIdx.x & (kWave - 1), hh = lane >> 5;
#pragma unroll
    for (int t = 0; t < 2; ++t) {
        const int k = min(k0 + 32 * t + (lane & 31), k_hi - 1);
        const u16* row = kv.krow_at((int)mod_magic((unsigned)k, (unsigned)kv.R, kv.magic));
#pragma unroll
        for (int kk = 0; kk < D / 16; ++kk)
            kr[t][kk] = __builtin_bit_cast(bf16x8, ld16(row + 16 * kk + 8 * hh));
    }
}

// This wave alone copies V rows [k0, k0 + 64) into its LDS tile (the layout
// of the workgroup copies: instruction i fills rows i*ROWS.., chunk c of row
// r at position c ^ swz(r)); rows at or past k_hi repeat row k_hi - 1.  The
// loads are non-temporal: a decode item reads its rows once (short step
// -1.5 %, benchmark table unchanged; the same on the compute items' copies
// cost the table 0.3 %, where q-blocks of one segment share key rows).
template <int D>
__device__ inline void copy_v_wave(const KVRing& kv, int k0, int k_hi, u16* dst) {
    constexpr int CH = D / 8, ROWS = 64 / CH, INSTR = kBN / ROWS;
    const int lane = threadIdx.x & (kWave - 1);
#pragma unroll
    for (int i = 0; i < INSTR; ++i) {
        const int r = i * ROWS + lane / CH;
        const int k = min(k0 + r, k_hi - 1);
        const int row = (int)mod_magic((unsigned)k, (unsigned)kv.R, kv.magic);
        __builtin_amdgcn_global_load_lds(
            (glb_void*)(kv.vb + (int64_t)row * kv.vs + 8 * ((lane % CH) ^ swz<D>(r))),
            (lds_void*)(dst + i * 512), 16, 0, 2);
    }
}

// The eight waves' 64-key V tiles of a decode item (the merge reuses them as
// fp32 buffers of the waves' accumulators).  Indexed with constants only.
struct WaveBufs {
    u16* b[kWaves];
};

// One decode item: kv head hk, split `split` of nsplit of the segment's
// visible keys, all q_len positions x gq heads as rows r = hl * q_len + pos.
template <int D>
__device__ __forceinline__ void decode_item(const VarlenArgs& a, const Segment& sg, int hk,
                                            int split, int nsplit, WaveBufs wb) {
    constexpr int NREG = (D / 32) * 16;  // accumulator floats per lane
    constexpr int RPW = NREG / kWaves;   // of which each wave merges
    __shared__ float sh_m[kWaves][32], sh_l[kWaves][32];
    const int gq = a.Hq / a.Hkv;
    const int lane = threadIdx.x & (kWave - 1), hh = lane >> 5;
    const int w = __builtin_amdgcn_readfirstlane(threadIdx.x / kWave);
    u16* vbuf = wb.b[0];
#pragma unroll
    for (int v = 1; v < kWaves; ++v) vbuf = w == v ? wb.b[v] : vbuf;
    const int r = lane & 31, hl = r / sg.q_len, pos = r % sg.q_len;
    const bool valid = r < gq * sg.q_len;
    const int t = sg.q_start + pos, h = hk * gq + hl;
    const int64_t base = (int64_t)sg.kv_end - sg.q_len;
    int64_t lo64, hi64, p_min, p_max;
    block_range(sg, 0, sg.q_len, &lo64, &hi64, &p_min, &p_max);
    const int64_t p_lane = valid ? base + pos : p_max;
    int k_lo, k_hi;
    split_range((int)lo64, (int)hi64, split, nsplit, &k_lo, &k_hi);

    bf16x8 qf[1][D / 16];
    load_q<D, false>(qf[0], a.q + (int64_t)t * a.qs[0] + (int64_t)h * a.qs[1], valid,
                     a.negate ? -a.c : a.c);
    const float c = a.c;
    const KVRing kv{a.k + (int64_t)sg.col * a.ks[1] + (int64_t)hk * a.ks[2],
                    a.v + (int64_t)sg.col * a.vs[1] + (int64_t)hk * a.vs[2], a.ks[0], a.vs[0],
                    sg.R, 0xFFFFFFFFu / (unsigned)sg.R};
    const LaneBounds lb = lane_bounds(k_lo, k_hi, sg.causal, sg.window, p_lane);
    RowState<D> st;
    init_state<D>(st);
    const int n = (k_hi - k_lo + kBN - 1) / kBN;
    for (int tile = w; tile < n; tile += kWaves) {
        const int k0 = k_lo + tile * kBN;
        copy_v_wave<D>(kv, k0, k_hi, vbuf);
        bf16x8 kr[2][D / 16];
        load_k_regs<D>(kr, kv, k0, k_hi);
        __builtin_amdgcn_s_waitcnt(0x0F70);  // vmcnt(0): K registers and the V tile
        TileScores S;
        S[0][0] = S[0][1] = f32x16{};
#pragma unroll
        for (int kk = 0; kk < D / 16; ++kk) {
            S[0][0] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kr[0][kk], qf[0][kk], S[0][0], 0, 0, 0);
            S[0][1] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kr[1][kk], qf[0][kk], S[0][1], 0, 0, 0);
        }
        mask_tile(S, k0, &lb);
        float alpha[1], lsum[1];
        update_max(S, c, st.m, alpha);
        rescale<D>(alpha, st);
        TileP pk;
        softmax_tile(S, c, st.m, pk, lsum);
        st.l[0] += lsum[0];
        pv_tile<D>(vbuf, pk, st, NoCopy{});
    }

    // merge: M = max of the waves' maxima, each wave's share scaled by
    // 2^((m_w - M) c), then summed over the waves element by element
    const float lw = sum_across_halves(st.l[0]);
    if (lane < 32) {
        sh_m[w][lane] = st.m[0];
        sh_l[w][lane] = lw;
    }
    __syncthreads();
    float M = -INFINITY;
#pragma unroll
    for (int v = 0; v < kWaves; ++v) M = __builtin_fmaxf(M, sh_m[v][r]);
    const float mref = M == -INFINITY ? 0.f : M;
    float L = 0.f;
#pragma unroll
    for (int v = 0; v < kWaves; ++v) {
        const float mv = sh_m[v][r];
        L += mv == -INFINITY ? 0.f : sh_l[v][r] * __builtin_amdgcn_exp2f((mv - mref) * c);
    }
    const float fw = st.m[0] == -INFINITY ? 0.f : __builtin_amdgcn_exp2f((st.m[0] - mref) * c);
    float* ob = reinterpret_cast<float*>(vbuf);
#pragma unroll
    for (int dt = 0; dt < D / 32; ++dt)
#pragma unroll
        for (int i = 0; i < 16; ++i) ob[(dt * 16 + i) * kWave + lane] = st.o[0][dt][i] * fw;
    __syncthreads();
    float acc[RPW];
#pragma unroll
    for (int j = 0; j < RPW; ++j) acc[j] = 0.f;
#pragma unroll
    for (int v = 0; v < kWaves; ++v) {
        const float* obv = reinterpret_cast<const float*>(wb.b[v]);
#pragma unroll
        for (int j = 0; j < RPW; ++j) acc[j] += obv[(w * RPW + j) * kWave + lane];
    }
    // a split partial takes the format of store_partial: the row's largest
    // |value| over all waves (each holds RPW of a lane's registers) sets the
    // power-of-two scale
    int e = 0;
    if (nsplit > 1) {
        __shared__ float sh_x[kWaves][32];
        float mx = 0.f;
#pragma unroll
        for (int j = 0; j < RPW; ++j) mx = __builtin_fmaxf(mx, __builtin_fabsf(acc[j]));
        mx = max_across_halves(mx);
        if (lane < 32) sh_x[w][lane] = mx;
        __syncthreads();
        mx = 0.f;
#pragma unroll
        for (int v = 0; v < kWaves; ++v) mx = __builtin_fmaxf(mx, sh_x[v][r]);
        (void)frexpf(L > 0.f ? mx / L : 0.f, &e);
        e = e < -100 ? -100 : (e > 127 ? 127 : e);
    }
    if (!valid) return;
    // register ri = dt*16 + i of a lane holds d = 32dt + 8(i/4) + 4hh + i%4
    if (nsplit == 1) {
        const float inv = L > 0.f ? 1.f / L : 0.f;
        u16* orow = a.out + (int64_t)t * a.os[0] + (int64_t)h * a.os[1];
#pragma unroll
        for (int j = 0; j < RPW; j += 4) {
            const int ri = w * RPW + j, dt = ri / 16, i = ri % 16;
            const int d = 32 * dt + 8 * (i / 4) + 4 * hh;
            *reinterpret_cast<uint2*>(orow + d) =
                make_uint2(pack_bf16x2(acc[j] * inv, acc[j + 1] * inv),
                           pack_bf16x2(acc[j + 2] * inv, acc[j + 3] * inv));
        }
    } else {
        const int64_t row = ((int64_t)t * a.Hq + h) * a.nsplit + split;
        u16* po = a.part_o + row * D;
        const float sc = ldexpf(L > 0.f ? 1.f / L : 0.f, -e);
#pragma unroll
        for (int j = 0; j < RPW; j += 4) {
            const int ri = w * RPW + j, dt = ri / 16, i = ri % 16;
            const int d = 32 * dt + 8 * (i / 4) + 4 * hh;
            *reinterpret_cast<uint2*>(po + d) =
                make_uint2(pack_f16x2(acc[j] * sc, acc[j + 1] * sc),
                           pack_f16x2(acc[j + 2] * sc, acc[j + 3] * sc));
        }
        if (w == 0 && hh == 0)
            *reinterpret_cast<float4*>(a.part_ml + row * 4) =
                make_float4(L > 0.f ? mref * c : -INFINITY, L, ldexpf(L, e), 0.f);
    }
}

template <int D>
__global__ __launch_bounds__(kThreads) void varlen_kernel(VarlenArgs a) {
    DECLARE_TILE_SMEM(D);
    const ClockMark cm = clock_mark(a.clk);

    const int g = a.Hq / a.Hkv;
    const RowMap rm = row_map(g);
    const int hg = a.Hkv * rm.hchunks;

    // this workgroup's work item: (segment, item j of that segment)
    int seg, j, sk = a.split_keys;
    Segment sg;
    const bool got = a.S <= kWave ? pick_item_wave(a, rm.P, hg, g, blockIdx.x, &j, &sg, &sk)
                                  : pick_item(a, rm.P, hg, g, blockIdx.x, &seg, &j, &sg);
    if (!got) return;
    const SegPlan pl = seg_plan(sg, rm.P, hg, g, a.Hkv, sk, a.nsplit);
    if (pl.decode) {
        __shared__ __attribute__((aligned(1024))) u16 sx[2 * kBN * D];
        WaveBufs wb;
        wb.b[0] = sk0;
        wb.b[1] = sv0;
        wb.b[2] = sk1;
        wb.b[3] = sv1;
        wb.b[4] = sk2;
        wb.b[5] = sv2;
        wb.b[6] = sx;
        wb.b[7] = sx + kBN * D;
        decode_item<D>(a, sg, j % a.Hkv, j / a.Hkv, pl.nsplit, wb);
        clock_add(a.clk, cm);
        return;
    }
    // item j: q-blocks from the last (the longest under causal masking),
    // then split, then (kv head, head chunk)
    const int per_qb = hg * pl.nsplit;
    const int qb = pl.nqb - 1 - j / per_qb;
    const int split = (j % per_qb) / hg, hy = j % hg;
    const int hk = hy / rm.hchunks, hc = hy % rm.hchunks;
    const int nsplit = pl.nsplit;
    int64_t lo64, hi64, p_min, p_max;
    block_range(sg, qb, rm.P, &lo64, &hi64, &p_min, &p_max);

    const int heads_here = min(rm.Gc, g - hc * rm.Gc);
    const int wave = threadIdx.x / kWave, lane = threadIdx.x & (kWave - 1);
    const int64_t base = (int64_t)sg.kv_end - sg.q_len;

    int hrow[kNT], jrow[kNT];
    bool valid[kNT];
    int64_t p_lane[kNT];
    bf16x8 qf[kNT][D / 16];
#pragma unroll
    for (int nt = 0; nt < kNT; ++nt) {
        const int r = (wave * kNT + nt) * 32 + (lane & 31);
        const int hl = r / rm.P, pos = r % rm.P;
        jrow[nt] = qb * rm.P + pos;
        hrow[nt] = hk * g + hc * rm.Gc + hl;
        valid[nt] = hl < heads_here && jrow[nt] < sg.q_len;
        p_lane[nt] = valid[nt] ? base + jrow[nt] : p_max;
        load_q<D, false>(qf[nt],
                         a.q + (int64_t)(sg.q_start + jrow[nt]) * a.qs[0] +
                             (int64_t)hrow[nt] * a.qs[1],
                         valid[nt], a.negate ? -a.c : a.c);
    }

    int k_lo, k_hi;
    split_range((int)lo64, (int)hi64, split, nsplit, &k_lo, &k_hi);

    RowState<D> st;
    init_state<D>(st);
    KVRing kv{a.k + (int64_t)sg.col * a.ks[1] + (int64_t)hk * a.ks[2],
              a.v + (int64_t)sg.col * a.vs[1] + (int64_t)hk * a.vs[2], a.ks[0], a.vs[0], sg.R,
              0xFFFFFFFFu / (unsigned)sg.R};
    const bool redone =
        attend<D, false>(kv, k_lo, k_hi, sg.causal, sg.window, p_lane, p_min, p_max, qf, a.c, st, sm);

    u16* const tile = row_tile<D>(sm, __builtin_amdgcn_readfirstlane(wave));
    __syncthreads();  // every wave is done with the stages
    const int t = sg.q_start + jrow[0];
    if (nsplit == 1) {
        store_out<D>(st.o[0], st.l[0], a.out + (int64_t)t * a.os[0] + (int64_t)hrow[0] * a.os[1],
                     valid[0], tile);
    } else {
        const int64_t row = ((int64_t)t * a.Hq + hrow[0]) * a.nsplit + split;
        store_partial<D>(st.o[0], st.m[0], st.l[0], a.c, a.part_o + row * D, a.part_ml + row * 4,
                         valid[0], tile);
    }
    clock_add(a.clk, cm, redone);
}

// Finish pass, one packed row per workgroup: merge split partials, zero a
// row that no valid segment covers, and record this workgroup's error word
// (workgroup 0 also reports every segment's flags).  With at most 64
// segments each wave finds the row's segments on its own (lane s checks
// segment s; the lowest covering one owns the row); else through LDS.  G:
// splits whose loads are in flight together: 16 for few packed rows, where
// the extra registers cost no residency; otherwise 4, whose 57 registers
// let 8 waves share a SIMD, so a table of ~2000 rows is resident at once
// (most rows have at most 4 splits).
template <int D, int G>
__global__ __launch_bounds__(256) void varlen_finish_kernel(VarlenArgs a) {
    const int g = a.Hq / a.Hkv;
    const RowMap rm = row_map(g);
    const int t = blockIdx.x;
    int flags = 0, owner = -1, count = 0, ns = 1;
    if (a.S <= kWave) {
        const int lane = threadIdx.x & (kWave - 1);
        const bool has = lane < a.S;
        const Segment x = has ? read_segment(a, lane) : Segment{};
        const bool cov = has && !x.flags && t < a.T && t >= x.q_start && t < x.q_start + x.q_len;
        const int hg = a.Hkv * rm.hchunks;
        SegPlan px;
        if (a.adaptive)
            (void)choose_split_wave(a, x, has, rm.P, hg, g, &px);
        else
            px = has ? seg_plan(x, rm.P, hg, g, a.Hkv, a.split_keys, a.nsplit)
                     : SegPlan{0, 1, 0, 0, false};
        const uint64_t m = __ballot(cov);
        count = __builtin_popcountll(m);
        if (m) {
            owner = __builtin_ctzll(m);
            const int my_ns = cov ? px.nsplit : 1;
            ns = __builtin_amdgcn_readlane(my_ns, owner);
        }
        if (blockIdx.x == 0)
            for (int b = 1; b <= ATTN_SEG_SPAN; b <<= 1) flags |= __ballot(x.flags & b) ? b : 0;
    } else {
        __shared__ int flags_sh, owner_sh, count_sh, ns_sh;
        if (threadIdx.x == 0) {
            flags_sh = 0;
            owner_sh = 0x7fffffff;
            count_sh = 0;
        }
        __syncthreads();
        int fl = 0, mine = -1, my_ns = 1;
        for (int s = threadIdx.x; s < a.S; s += 256) {
            const Segment x = read_segment(a, s);
            if (blockIdx.x == 0) fl |= x.flags;
            if (!x.flags && t < a.T && t >= x.q_start && t < x.q_start + x.q_len) {
                atomicMin(&owner_sh, s);
                atomicAdd(&count_sh, 1);
                if (mine < 0) {  // this thread's first (lowest) covering segment
                    mine = s;
                    my_ns = seg_plan(x, rm.P, a.Hkv * rm.hchunks, g, a.Hkv, a.split_keys, a.nsplit)
                                .nsplit;
                }
            }
        }
        if (fl) atomicOr(&flags_sh, fl);
        __syncthreads();
        // the thread that read the owning segment publishes its split count
        if (mine >= 0 && mine == owner_sh) ns_sh = my_ns;
        __syncthreads();
        flags = flags_sh;
        count = count_sh;
        owner = owner_sh == 0x7fffffff ? -1 : owner_sh;
        ns = owner >= 0 ? ns_sh : 1;
    }
    if (t < a.T && (owner < 0 || ns > 1)) {
        constexpr int TPR = D / 8;  // threads per (row, head), 8 dims each
        for (int e = threadIdx.x; e < a.Hq * TPR; e += 256) {
            const int h = e / TPR, d0 = (e % TPR) * 8;
            u16* orow = a.out + (int64_t)t * a.os[0] + (int64_t)h * a.os[1];
            if (owner < 0) {
                *reinterpret_cast<uint4*>(orow + d0) = make_uint4(0, 0, 0, 0);
            } else {
                const int64_t row = ((int64_t)t * a.Hq + h) * a.nsplit;
                combine_row<D, G>(a.part_o + row * D, a.part_ml + row * 4, D, 4, ns, d0, orow);
            }
        }
    }
    if (threadIdx.x == 0) a.err[blockIdx.x] = flags | (count > 1 ? ATTN_SEG_OVERLAP : 0);
}

// ---------------------------------------------------------------- slot write
//
// The step's new K/V rows go to row position mod R of their sequence's
// column ("[executorch][cuda] Add a length-aware Triton SDPA over
// per-sequence KV columns": the batched-sequence manifest layout writes slot
// (position mod rows) x columns + column; the batched sequence cache gives
// each sequence a column, a scratch last column, and ring layers of R rows).
// One wave per token copies its Hkv x D values of K and of V in 16-byte
// pieces; four tokens per workgroup, whose flags form its error word.

struct KVWriteArgs {
    const u16* kn;
    const u16* vn;
    u16* ks;
    u16* vs;
    const int64_t* pos;
    const int32_t* col;
    const int32_t* srows;  // per-token modulus (<= 0: rows), or null
    int32_t* err;          // one word per workgroup
    int T, Hkv, D, rows, cols;
    int64_t kns[3], vns[3], kss[4], vss[4];
};

constexpr int kWriteTokens = 4;  // tokens (waves) per slot-write workgroup

__global__ __launch_bounds__(kWriteTokens * kWave) void kv_write_kernel(KVWriteArgs a) {
    __shared__ int flags_sh;
    const int lane = threadIdx.x & (kWave - 1);
    const int i = blockIdx.x * kWriteTokens + (int)(threadIdx.x / kWave);
    if (threadIdx.x == 0) flags_sh = 0;
    __syncthreads();
    int f = 0;
    if (i < a.T) {
        const int64_t p = a.pos[i];
        const int c = a.col[i];
        const int rr = a.srows ? a.srows[i] : 0;
        const int R = rr > 0 ? rr : a.rows;
        if (c < 0 || c >= a.cols) f |= ATTN_KV_COL;
        if (p < 0) f |= ATTN_KV_POS;
        if (R > a.rows) f |= ATTN_KV_ROWS;
        if (!f) {
            const int64_t r = p % R;
            const int per_head = a.D / 8;  // 16-byte pieces of one head's row
            for (int e = lane; e < a.Hkv * per_head; e += kWave) {
                const int h = e / per_head, d = (e % per_head) * 8;
                const uint4 kx = ld16(a.kn + i * a.kns[0] + h * a.kns[1] + d);
                const uint4 vx = ld16(a.vn + i * a.vns[0] + h * a.vns[1] + d);
                *reinterpret_cast<uint4*>(a.ks + r * a.kss[0] + c * a.kss[1] + h * a.kss[2] + d) = kx;
                *reinterpret_cast<uint4*>(a.vs + r * a.vss[0] + c * a.vss[1] + h * a.vss[2] + d) = vx;
            }
        } else if (lane == 0) {
            atomicOr(&flags_sh, f);
        }
    }
    __syncthreads();
    if (threadIdx.x == 0) a.err[blockIdx.x] = flags_sh;
}

// ---------------------------------------------------------------- host side

thread_local char g_err[512];

int fail(int code, const char* fmt, ...) __attribute__((format(printf, 2, 3)));
int fail(int code, const char* fmt, ...) {
    va_list ap;
    va_start(ap, fmt);
    vsnprintf(g_err, sizeof g_err, fmt, ap);
    va_end(ap);
    return code;
}

void clear_err() { g_err[0] = 0; }

// Optional timing of the attention kernels (attn_timing_begin / _end): HIP
// event pairs recorded on the launch stream around each attention kernel,
// per host thread.  Events are reused across begin/end rounds.
struct Timing {
    bool on = false;
    int dev = -1;                      // device current at attn_timing_begin
    unsigned long long* clk = nullptr; // its g_clock, when it could be cleared
    std::vector<std::pair<hipEvent_t, hipEvent_t>> marks;
    std::vector<hipEvent_t> pool;
    hipEvent_t get() {
        if (!pool.empty()) {
            hipEvent_t e = pool.back();
            pool.pop_back();
            return e;
        }
        hipEvent_t e = nullptr;
        return hipEventCreate(&e) == hipSuccess ? e : nullptr;
    }
    void recycle() {
        for (auto& m : marks) {
            if (m.first) pool.push_back(m.first);
            if (m.second) pool.push_back(m.second);
        }
        marks.clear();
    }
};
thread_local Timing g_timing;

// Records the start event of a timed launch (nullptr when timing is off).
hipEvent_t timing_start(hipStream_t s) {
    if (!g_timing.on) return nullptr;
    hipEvent_t e = g_timing.get();
    if (e && hipEventRecord(e, s) != hipSuccess) e = nullptr;
    return e;
}

// Clock sums for a kernel launched now on the current device (null when
// timing is off or the device is not the one timing began on).
unsigned long long* timing_clock() {
    int dev = -1;
    if (!g_timing.on || !g_timing.clk || hipGetDevice(&dev) != hipSuccess) return nullptr;
    return dev == g_timing.dev ? g_timing.clk : nullptr;
}

void timing_stop(hipEvent_t start, hipStream_t s) {
    if (!start) return;
    hipEvent_t e = g_timing.get();
    if (e && hipEventRecord(e, s) != hipSuccess) e = nullptr;
    g_timing.marks.push_back({start, e});
}

struct DeviceInfo {
    int cus;
    int prefill_per_cu[3];  // resident prefill workgroups per CU at D = 64, 128, 256
};

// Resident workgroups per CU of a kernel (the occupancy API; 1 if it cannot
// answer).
template <class K>
int resident_per_cu(K kernel, int threads) {
    int n = 0;
    if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&n, kernel, threads, 0) != hipSuccess || n < 1)
        n = 1;
    (void)hipGetLastError();
    return n;
}

constexpr int kMaxDevices = 64;
std::once_flag g_dev_once[kMaxDevices];
DeviceInfo g_dev[kMaxDevices];

int device_info(DeviceInfo* out) {
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices)
        return fail(ATTN_ERR_HIP, "hipGetDevice failed");
    std::call_once(g_dev_once[dev], [dev] {
        int cus = 0;
        if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess)
            cus = 0;
        g_dev[dev].cus = cus;
        // the fewer of the two variants' (scale in Q or not)
        g_dev[dev].prefill_per_cu[0] = std::min(resident_per_cu(prefill_kernel<64, true>, kThreads),
                                                resident_per_cu(prefill_kernel<64, false>, kThreads));
        g_dev[dev].prefill_per_cu[1] =
            std::min(resident_per_cu(prefill_kernel<128, true>, kThreads),
                     resident_per_cu(prefill_kernel<128, false>, kThreads));
        g_dev[dev].prefill_per_cu[2] =
            std::min(resident_per_cu(prefill256_kernel<true>, kWaves256 * kWave),
                     resident_per_cu(prefill256_kernel<false>, kWaves256 * kWave));
    });
    if (g_dev[dev].cus <= 0) return fail(ATTN_ERR_HIP, "could not read the compute-unit count");
    *out = g_dev[dev];
    return ATTN_OK;
}

int env_int(const char* name, int dflt) {
    const char* s = getenv(name);
    if (!s || !*s) return dflt;
    return atoi(s);
}

constexpr int64_t kMaxOffset = (int64_t)1 << 62;

// Largest element offset reachable through sizes/strides (strides >= 0).
bool offset_ok(const int64_t* sizes, const int64_t* str, int n) {
    __int128 m = 0;
    for (int i = 0; i < n; ++i) {
        if (sizes[i] <= 0) return true;
        m += (__int128)(sizes[i] - 1) * str[i];
    }
    return m < kMaxOffset;
}

// Layout rules shared by every tensor argument: innermost stride 1, other
// strides non-negative multiples of 8 elements, 16-byte aligned base.
int check_layout(const char* name, const void* p, const int64_t* str, int n) {
    if (str[n - 1] != 1)
        return fail(ATTN_ERR_UNSUPPORTED, "%s: innermost stride %lld, only 1 is supported", name,
                    (long long)str[n - 1]);
    for (int i = 0; i < n - 1; ++i)
        if (str[i] < 0 || str[i] % 8 != 0)
            return fail(ATTN_ERR_UNSUPPORTED,
                        "%s: stride[%d] = %lld is not a non-negative multiple of 8", name, i,
                        (long long)str[i]);
    if ((uintptr_t)p % 16 != 0)
        return fail(ATTN_ERR_UNSUPPORTED, "%s: base pointer is not 16-byte aligned", name);
    return ATTN_OK;
}

constexpr int64_t kMaxRowStride = (int64_t)1 << 24;

size_t align256(size_t x) { return (x + 255) / 256 * 256; }

// Key splits of a prefill launch: enough workgroups to fill every compute
// unit once (as many per CU as the occupancy API reports resident for the
// kernel: one for each head dimension's kernel today), with at least 1024
// keys per split.
int prefill_splits(int B, int Hq, int Hkv, int Lq, int Lkv, int D, const DeviceInfo& di) {
    const int cus = di.cus;
    int forced = env_int("ATTN_FORCE_SPLITS", 0);
    RowMap rm = row_map(Hq / Hkv, D == 256 ? kBM256 : kBM);
    int64_t base = (int64_t)((Lq + rm.P - 1) / rm.P) * rm.hchunks * B * Hkv;
    int by_keys = (Lkv + 1023) / 1024;
    if (by_keys < 1) by_keys = 1;
    int ns;
    if (forced > 0) {
        ns = forced;
    } else {
        const int per_cu = di.prefill_per_cu[D == 64 ? 0 : (D == 128 ? 1 : 2)];
        int64_t want = (per_cu * (int64_t)cus + base - 1) / (base > 0 ? base : 1);
        ns = (int)(want < kMaxSplits ? want : kMaxSplits);
        if (ns > by_keys) ns = by_keys;
    }
    if (ns < 1) ns = 1;
    if (ns > kMaxSplits) ns = kMaxSplits;
    return ns;
}

// Prefill split partials: fp16 values (D per row) and a 4-float record per row.
size_t prefill_ws_bytes(int B, int Hq, int Lq, int D, int nsplit) {
    if (nsplit <= 1) return 0;
    size_t rows = (size_t)nsplit * B * Hq * Lq;
    return align256(rows * D * sizeof(u16)) + align256(rows * 4 * sizeof(float));
}

// Target keys per split of a varlen q-block (ATTN_VARLEN_SPLIT_KEYS overrides,
// at least one 64-key tile), and the most splits of a q-block: enough for the
// longest range a flat column can hold.  A q-block of a longer range (ring
// storage) takes bigger chunks.
int varlen_split_keys() {
    int k = env_int("ATTN_VARLEN_SPLIT_KEYS", kVarlenSplitKeys);
    return k < kBN ? kBN : k;
}

int varlen_splits(int rows) {
    int forced = env_int("ATTN_FORCE_SPLITS", 0);
    const int keys = varlen_split_keys();
    int ns = forced > 0 ? forced : (rows + keys - 1) / keys;
    if (ns < 1) ns = 1;
    if (ns > kMaxVarlenSplits) ns = kMaxVarlenSplits;
    return ns;
}

int varlen_finish_blocks(int T) { return T > 0 ? T : 1; }

size_t varlen_ws_bytes(int S, int T, int Hq, int Hkv, int D, int rows) {
    (void)S;
    (void)Hkv;
    int ns = varlen_splits(rows);
    size_t bytes = align256((size_t)varlen_finish_blocks(T) * sizeof(int32_t));
    if (ns > 1) {
        size_t prow = (size_t)(T > 0 ? T : 0) * Hq * ns;
        bytes += align256(prow * D * sizeof(u16)) + align256(prow * 4 * sizeof(float));
    }
    return bytes;
}

// Device address of `scratch` on each device, taken once per device with
// that device current (each device holds its own copy of the array).
std::once_flag g_scratch_once[kMaxDevices];
void* g_scratch_ptr[kMaxDevices];

int scratch_address(void** out) {
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices)
        return fail(ATTN_ERR_HIP, "hipGetDevice failed");
    std::call_once(g_scratch_once[dev], [dev] {
        void* p = nullptr;
        if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess) {
            (void)hipGetLastError();
            p = nullptr;
        }
        g_scratch_ptr[dev] = p;
    });
    if (!g_scratch_ptr[dev]) return fail(ATTN_ERR_HIP, "could not read the scratch buffer's address");
    *out = g_scratch_ptr[dev];
    return ATTN_OK;
}

}  // namespace

extern "C" {

int attn_abi_version(void) { return 1; }

const char* attn_last_error(void) { return g_err; }

size_t attn_causal_prefill_workspace(int B, int Hq, int Hkv, int Lq, int Lkv, int D) {
    if (B < 1 || Hq < 1 || Hkv < 1 || Lq < 0 || Lkv < 0 || Hq % Hkv != 0) return 0;
    if (D != 64 && D != 128 && D != 256) return 0;
    if (Lq == 0) return 0;
    DeviceInfo di;
    if (device_info(&di) != ATTN_OK) return 0;
    return prefill_ws_bytes(B, Hq, Lq, D, prefill_splits(B, Hq, Hkv, Lq, Lkv, D, di));
}

// Both prefill entry points: with bounds (device (q_pos0, kv_len)), the
// workspace starts with the 256-byte error word and the partials follow.
static int prefill_call(const void* q, const void* k, const void* v, void* out, int B, int Hq, int Hkv,
                 int Lq, int Lkv, int D, float scale, const int64_t q_str[4],
                 const int64_t k_str[4], const int64_t v_str[4], const int64_t o_str[4],
                 int64_t q_pos0, const int64_t* bounds, int window, void* workspace,
                 size_t ws_bytes, void* stream, bool use_scratch = false) {
    clear_err();
    if (!q_str || !k_str || !v_str || !o_str) return fail(ATTN_ERR_INVALID, "null stride array");
    if (B < 1 || Hq < 1 || Hkv < 1 || Lq < 0 || Lkv < 0)
        return fail(ATTN_ERR_INVALID, "sizes must satisfy B,Hq,Hkv >= 1 and Lq,Lkv >= 0");
    // empty tensors may come with null pointers
    if ((Lq > 0 && (!q || !out)) || (Lkv > 0 && (!k || !v)))
        return fail(ATTN_ERR_INVALID, "null tensor pointer");
    if (Hq % Hkv != 0) return fail(ATTN_ERR_INVALID, "Hq (%d) is not a multiple of Hkv (%d)", Hq, Hkv);
    if (!(scale == scale) || isinf(scale)) return fail(ATTN_ERR_INVALID, "scale is not finite");
    if (D != 64 && D != 128 && D != 256)
        return fail(ATTN_ERR_UNSUPPORTED, "head dim %d: only 64, 128 and 256", D);
    if (q_pos0 > kMaxOffset || q_pos0 < -kMaxOffset)
        return fail(ATTN_ERR_INVALID, "q_pos0 out of range");
    int st;
    if ((st = check_layout("q", q, q_str, 4))) return st;
    if ((st = check_layout("k", k, k_str, 4))) return st;
    if ((st = check_layout("v", v, v_str, 4))) return st;
    if ((st = check_layout("out", out, o_str, 4))) return st;
    // tile copies address the rows of a 64-key tile with 32-bit byte offsets
    if (k_str[2] >= kMaxRowStride || v_str[2] >= kMaxRowStride)
        return fail(ATTN_ERR_UNSUPPORTED, "k/v row stride must be below 2^24 elements");
    const int64_t qsz[4] = {B, Hq, Lq, D}, ksz[4] = {B, Hkv, Lkv, D};
    if (!offset_ok(qsz, q_str, 4) || !offset_ok(ksz, k_str, 4) || !offset_ok(ksz, v_str, 4) ||
        !offset_ok(qsz, o_str, 4))
        return fail(ATTN_ERR_INVALID, "element offsets exceed 2^62");
    if (bounds && (uintptr_t)bounds % 8 != 0)
        return fail(ATTN_ERR_UNSUPPORTED, "bounds is not 8-byte aligned");
    if (Lq == 0) return ATTN_OK;

    DeviceInfo di;
    if ((st = device_info(&di))) return st;
    const int nsplit = prefill_splits(B, Hq, Hkv, Lq, Lkv, D, di);
    const size_t errb = bounds ? 256 : 0;
    const size_t need = errb + prefill_ws_bytes(B, Hq, Lq, D, nsplit);
    if (use_scratch && need > 0) {
        // the partials go to the static buffer instead of a caller workspace
        if (need > (size_t)ATTN_NOALLOC_SCRATCH_BYTES)
            return fail(ATTN_ERR_WORKSPACE,
                        "split partials of %zu bytes exceed the %zu-byte static scratch buffer "
                        "(call attn_causal_prefill with a workspace instead)",
                        need, (size_t)ATTN_NOALLOC_SCRATCH_BYTES);
        if ((st = scratch_address(&workspace))) return st;
        ws_bytes = (size_t)ATTN_NOALLOC_SCRATCH_BYTES;
    }
    if (need > 0 && (!workspace || ws_bytes < need))
        return fail(ATTN_ERR_WORKSPACE, "workspace of %zu bytes needed, %zu given", need,
                    workspace ? ws_bytes : (size_t)0);
    if (need > 0 && (uintptr_t)workspace % 256 != 0)
        return fail(ATTN_ERR_WORKSPACE, "workspace is not 256-byte aligned");

    PrefillArgs a;
    a.q = (const u16*)q;
    a.k = (const u16*)k;
    a.v = (const u16*)v;
    a.out = (u16*)out;
    size_t prow = (size_t)nsplit * B * Hq * Lq;
    const bool parts = need > errb;
    a.part_o = parts ? (u16*)((char*)workspace + errb) : nullptr;
    a.part_ml =
        parts ? (float*)((char*)workspace + errb + align256(prow * D * sizeof(u16))) : nullptr;
    a.bounds = bounds;
    a.err = bounds ? (int32_t*)workspace : nullptr;
    a.B = B;
    a.Hq = Hq;
    a.Hkv = Hkv;
    a.Lq = Lq;
    a.Lkv = Lkv;
    a.window = window > 0 ? window : 0;
    a.nsplit = nsplit;
    // c > 0 keeps exp2(-inf * c) = 0 for masked scores; a zero scale gives
    // weights that round to exactly 1 (uniform)
    a.c = fmaxf(fabsf(scale) * kLog2e, 1e-30f);
    a.negate = scale < 0.f;
    a.q_pos0 = q_pos0;
    for (int i = 0; i < 4; ++i) {
        a.qs[i] = q_str[i];
        a.ks[i] = k_str[i];
        a.vs[i] = v_str[i];
        a.os[i] = o_str[i];
    }
    RowMap rm = row_map(Hq / Hkv, D == 256 ? kBM256 : kBM);
    const int64_t n_inner = (int64_t)((Lq + rm.P - 1) / rm.P) * rm.hchunks;
    const int64_t nwg = n_inner * B * Hkv * nsplit;
    if (nwg > 0x7fffffff)
        return fail(ATTN_ERR_UNSUPPORTED, "launch grid too large (%lld workgroups)", (long long)nwg);
    a.n_inner = (int)n_inner;
    hipStream_t s = (hipStream_t)stream;
    dim3 grid((unsigned)nwg);
    a.clk = timing_clock();
    // The scale goes into Q (rounded to bf16 with it) when |scale| <= 1/sqrt(D),
    // the standard scale and below: there that rounding moves the scores by
    // no more than it does at the standard scale.  A larger scale sharpens
    // the softmax and would magnify it, so Q stays exact and the softmax
    // multiplies by the scale in fp32.
    const bool ps = fabsf(scale) * sqrtf((float)D) <= 1.0001f;
    hipEvent_t t0 = timing_start(s);
    if (D == 64) {
        if (ps)
            hipLaunchKernelGGL((prefill_kernel<64, true>), grid, dim3(kThreads), 0, s, a);
        else
            hipLaunchKernelGGL((prefill_kernel<64, false>), grid, dim3(kThreads), 0, s, a);
    } else if (D == 128) {
        if (ps)
            hipLaunchKernelGGL((prefill_kernel<128, true>), grid, dim3(kThreads), 0, s, a);
        else
            hipLaunchKernelGGL((prefill_kernel<128, false>), grid, dim3(kThreads), 0, s, a);
    } else {
        if (ps)
            hipLaunchKernelGGL(prefill256_kernel<true>, grid, dim3(kWaves256 * kWave), 0, s, a);
        else
            hipLaunchKernelGGL(prefill256_kernel<false>, grid, dim3(kWaves256 * kWave), 0, s, a);
    }
    timing_stop(t0, s);
    if (hipGetLastError() != hipSuccess) return fail(ATTN_ERR_HIP, "prefill launch failed");
    if (nsplit > 1) {
        int64_t rows = (int64_t)B * Hq * Lq;
        int per = 256 / (D / 8);  // rows per combine workgroup
        int64_t nb = (rows + per - 1) / per;
        if (D == 64)
            hipLaunchKernelGGL(prefill_combine_kernel<64>, dim3((unsigned)nb), dim3(256), 0, s, a);
        else if (D == 128)
            hipLaunchKernelGGL(prefill_combine_kernel<128>, dim3((unsigned)nb), dim3(256), 0, s, a);
        else
            hipLaunchKernelGGL(prefill_combine_kernel<256>, dim3((unsigned)nb), dim3(256), 0, s, a);
        if (hipGetLastError() != hipSuccess) return fail(ATTN_ERR_HIP, "combine launch failed");
    }
    return ATTN_OK;
}

int attn_causal_prefill(const void* q, const void* k, const void* v, void* out, int B, int Hq,
                        int Hkv, int Lq, int Lkv, int D, float scale, const int64_t q_str[4],
                        const int64_t k_str[4], const int64_t v_str[4], const int64_t o_str[4],
                        int64_t q_pos0, int window, void* workspace, size_t ws_bytes,
                        void* stream) {
    return prefill_call(q, k, v, out, B, Hq, Hkv, Lq, Lkv, D, scale, q_str, k_str, v_str, o_str,
                        q_pos0, nullptr, window, workspace, ws_bytes, stream);
}

int attn_causal_prefill_noalloc(const void* q, const void* k, const void* v, void* out, int B,
                                int Hq, int Hkv, int Lq, int Lkv, int D, float scale,
                                const int64_t q_str[4], const int64_t k_str[4],
                                const int64_t v_str[4], const int64_t o_str[4], int64_t q_pos0,
                                int window, void* stream) {
    return prefill_call(q, k, v, out, B, Hq, Hkv, Lq, Lkv, D, scale, q_str, k_str, v_str, o_str,
                        q_pos0, nullptr, window, nullptr, 0, stream, true);
}

size_t attn_causal_prefill_dev_workspace(int B, int Hq, int Hkv, int Lq, int Lkv, int D) {
    if (B < 1 || Hq < 1 || Hkv < 1 || Lq < 0 || Lkv < 0 || Hq % Hkv != 0) return 0;
    if (D != 64 && D != 128 && D != 256) return 0;
    return 256 + attn_causal_prefill_workspace(B, Hq, Hkv, Lq, Lkv, D);
}

int attn_causal_prefill_dev(const void* q, const void* k, const void* v, void* out, int B,
                            int Hq, int Hkv, int Lq, int Lkv, int D, float scale,
                            const int64_t q_str[4], const int64_t k_str[4],
                            const int64_t v_str[4], const int64_t o_str[4],
                            const int64_t* bounds, int window, void* workspace, size_t ws_bytes,
                            void* stream) {
    if (!bounds) {
        clear_err();
        return fail(ATTN_ERR_INVALID, "null bounds");
    }
    if (Lq > 0 && (!workspace || ws_bytes < 256)) {
        clear_err();
        return fail(ATTN_ERR_WORKSPACE, "workspace of at least 256 bytes needed");
    }
    return prefill_call(q, k, v, out, B, Hq, Hkv, Lq, Lkv, D, scale, q_str, k_str, v_str, o_str,
                        0, bounds, window, workspace, ws_bytes, stream);
}

int attn_prefill_read_error(const void* workspace, void* stream, int32_t* err_out) {
    clear_err();
    if (!workspace || !err_out) return fail(ATTN_ERR_INVALID, "null pointer");
    if (hipStreamSynchronize((hipStream_t)stream) != hipSuccess)
        return fail(ATTN_ERR_HIP, "stream sync failed");
    if (hipMemcpy(err_out, workspace, sizeof(int32_t), hipMemcpyDeviceToHost) != hipSuccess)
        return fail(ATTN_ERR_HIP, "copy of the error word failed");
    return ATTN_OK;
}

size_t attn_sdpa_varlen_workspace(int S, int T, int Hq, int Hkv, int D, int rows, int cols) {
    if (S < 0 || T < 0 || Hq < 1 || Hkv < 1 || Hq % Hkv != 0 || rows < 1 || cols < 2) return 0;
    if (D != 64 && D != 128) return 0;
    return varlen_ws_bytes(S, T, Hq, Hkv, D, rows);
}

int attn_sdpa_varlen(const void* q, const void* k_store, const void* v_store, void* out,
                     const int32_t* seq_info, int S, const int32_t* seg_attr, int T, int Hq,
                     int Hkv, int D, int rows, int cols, float scale, int causal, int window,
                     int ring_rows, const int64_t q_str[3], const int64_t k_str[4],
                     const int64_t v_str[4], const int64_t o_str[3], void* workspace,
                     size_t ws_bytes, void* stream) {
    clear_err();
    if (!k_store || !v_store || (T > 0 && (!q || !out)))
        return fail(ATTN_ERR_INVALID, "null tensor pointer");
    if (!q_str || !k_str || !v_str || !o_str) return fail(ATTN_ERR_INVALID, "null stride array");
    if (S < 0 || T < 0 || Hq < 1 || Hkv < 1 || rows < 1 || cols < 2)
        return fail(ATTN_ERR_INVALID,
                    "sizes must satisfy S,T >= 0, Hq,Hkv,rows >= 1 and cols >= 2");
    if (S > 0 && !seq_info) return fail(ATTN_ERR_INVALID, "null seq_info");
    if (Hq % Hkv != 0) return fail(ATTN_ERR_INVALID, "Hq (%d) is not a multiple of Hkv (%d)", Hq, Hkv);
    if ((int64_t)S > 2 * (int64_t)(cols - 1))
        return fail(ATTN_ERR_INVALID, "S = %d exceeds 2 x (cols - 1) = %d segments", S,
                    2 * (cols - 1));
    if (!seg_attr && ring_rows > rows)
        return fail(ATTN_ERR_INVALID, "ring_rows %d exceeds rows %d", ring_rows, rows);
    if (!seg_attr && !causal && window > 0)
        return fail(ATTN_ERR_INVALID, "a window needs causal attention");
    if (!(scale == scale) || isinf(scale)) return fail(ATTN_ERR_INVALID, "scale is not finite");
    if (D != 64 && D != 128) return fail(ATTN_ERR_UNSUPPORTED, "head dim %d: only 64 and 128", D);
    int st;
    if ((st = check_layout("q", q, q_str, 3))) return st;
    if ((st = check_layout("k_store", k_store, k_str, 4))) return st;
    if ((st = check_layout("v_store", v_store, v_str, 4))) return st;
    if ((st = check_layout("out", out, o_str, 3))) return st;
    if (seq_info && (uintptr_t)seq_info % 4 != 0)
        return fail(ATTN_ERR_UNSUPPORTED, "seq_info is not 4-byte aligned");
    if (seg_attr && (uintptr_t)seg_attr % 4 != 0)
        return fail(ATTN_ERR_UNSUPPORTED, "seg_attr is not 4-byte aligned");
    const int64_t qsz[3] = {T, Hq, D}, ssz[4] = {rows, cols, Hkv, D};
    if (!offset_ok(qsz, q_str, 3) || !offset_ok(ssz, k_str, 4) || !offset_ok(ssz, v_str, 4) ||
        !offset_ok(qsz, o_str, 3))
        return fail(ATTN_ERR_INVALID, "element offsets exceed 2^62");
    const size_t need = varlen_ws_bytes(S, T, Hq, Hkv, D, rows);
    if (!workspace || ws_bytes < need)
        return fail(ATTN_ERR_WORKSPACE, "workspace of %zu bytes needed, %zu given", need,
                    workspace ? ws_bytes : (size_t)0);
    if ((uintptr_t)workspace % 256 != 0)
        return fail(ATTN_ERR_WORKSPACE, "workspace is not 256-byte aligned");
    DeviceInfo di;
    if ((st = device_info(&di))) return st;

    const int nsplit = varlen_splits(rows);
    RowMap rm = row_map(Hq / Hkv);
    VarlenArgs a;
    a.q = (const u16*)q;
    a.k = (const u16*)k_store;
    a.v = (const u16*)v_store;
    a.out = (u16*)out;
    a.seq_info = seq_info;
    a.seg_attr = seg_attr;
    a.err = (int32_t*)workspace;
    size_t errb = align256((size_t)varlen_finish_blocks(T) * sizeof(int32_t));
    a.part_o = nullptr;
    a.part_ml = nullptr;
    if (nsplit > 1) {
        const size_t prow = (size_t)T * Hq * nsplit;
        a.part_o = (u16*)((char*)workspace + errb);
        a.part_ml = (float*)((char*)workspace + errb + align256(prow * D * sizeof(u16)));
    }
    a.S = S;
    a.T = T;
    a.Hq = Hq;
    a.Hkv = Hkv;
    a.rows = rows;
    a.cols = cols;
    a.causal = causal ? 1 : 0;
    a.window = window;
    a.ring_rows = ring_rows;
    a.nsplit = nsplit;
    a.split_keys = varlen_split_keys();
    // c > 0 keeps exp2(-inf * c) = 0 for masked scores; a zero scale gives
    // weights that round to exactly 1 (uniform)
    a.c = fmaxf(fabsf(scale) * kLog2e, 1e-30f);
    a.negate = scale < 0.f;
    for (int i = 0; i < 3; ++i) {
        a.qs[i] = q_str[i];
        a.os[i] = o_str[i];
    }
    for (int i = 0; i < 4; ++i) {
        a.ks[i] = k_str[i];
        a.vs[i] = v_str[i];
    }
    hipStream_t s = (hipStream_t)stream;
    // q-block slots of any table: the q-blocks of segments that share no
    // packed row number at most T / P + S, each with Hkv x hchunks (kv head,
    // head chunk) pairs.  When the finest split could need more than two
    // rounds of workgroups, and the table has at most 64 segments (and no
    // split override), the split size is chosen per table on the device so
    // that its items fit a launch of one workgroup per compute unit, or per
    // slot when there are more slots (choose_split_wave); otherwise the
    // launch bounds the items at the finest split, nsplit per slot.
    const int64_t slots = ((int64_t)(T + rm.P - 1) / rm.P + S) * ((int64_t)Hkv * rm.hchunks);
    a.adaptive = S <= kWave && !getenv("ATTN_FORCE_SPLITS") && !getenv("ATTN_VARLEN_SPLIT_KEYS") &&
                 rows < (1 << 30) && slots * nsplit > 2 * (int64_t)di.cus;
    const int64_t gx = a.adaptive ? std::max<int64_t>(slots, di.cus) : slots * nsplit;
    if (gx > 0x7fffffff) return fail(ATTN_ERR_UNSUPPORTED, "launch grid too large");
    a.gx = (int)gx;
    if (gx > 0 && T > 0 && S > 0) {
        dim3 grid((unsigned)gx);
        a.clk = timing_clock();
        hipEvent_t t0 = timing_start(s);
        if (D == 64)
            hipLaunchKernelGGL(varlen_kernel<64>, grid, dim3(kThreads), 0, s, a);
        else
            hipLaunchKernelGGL(varlen_kernel<128>, grid, dim3(kThreads), 0, s, a);
        timing_stop(t0, s);
        if (hipGetLastError() != hipSuccess) return fail(ATTN_ERR_HIP, "varlen launch failed");
    }
    dim3 fgrid((unsigned)varlen_finish_blocks(T));
    // few packed rows: one finish workgroup per row fits the CUs at any
    // residency, so all 16 splits' loads can be in flight at once; many rows:
    // the narrow merge for residency
    const bool few = T <= 2 * di.cus;
    if (D == 64)
        hipLaunchKernelGGL((few ? varlen_finish_kernel<64, 16> : varlen_finish_kernel<64, 4>),
                           fgrid, dim3(256), 0, s, a);
    else
        hipLaunchKernelGGL((few ? varlen_finish_kernel<128, 16> : varlen_finish_kernel<128, 4>),
                           fgrid, dim3(256), 0, s, a);
    if (hipGetLastError() != hipSuccess) return fail(ATTN_ERR_HIP, "varlen finish launch failed");
    return ATTN_OK;
}

int attn_varlen_read_error(const void* workspace, int S, int T, void* stream, int32_t* err_out) {
    clear_err();
    if (!workspace || !err_out) return fail(ATTN_ERR_INVALID, "null pointer");
    if (S < 0 || T < 0) return fail(ATTN_ERR_INVALID, "negative size");
    (void)S;
    int n = varlen_finish_blocks(T);
    hipStream_t s = (hipStream_t)stream;
    if (hipStreamSynchronize(s) != hipSuccess) return fail(ATTN_ERR_HIP, "stream sync failed");
    int32_t* host = (int32_t*)malloc(sizeof(int32_t) * n);
    if (!host) return fail(ATTN_ERR_INVALID, "host allocation failed");
    if (hipMemcpy(host, workspace, sizeof(int32_t) * n, hipMemcpyDeviceToHost) != hipSuccess) {
        free(host);
        return fail(ATTN_ERR_HIP, "copy of the error word failed");
    }
    int32_t e = 0;
    for (int i = 0; i < n; ++i) e |= host[i];
    free(host);
    *err_out = e;
    return ATTN_OK;
}

static int kv_write_blocks(int T) { return T > 0 ? (T + kWriteTokens - 1) / kWriteTokens : 0; }

size_t attn_kv_write_workspace(int T) {
    if (T < 0) return 0;
    return align256((size_t)(kv_write_blocks(T) > 0 ? kv_write_blocks(T) : 1) * sizeof(int32_t));
}

int attn_kv_write(const void* k_new, const void* v_new, void* k_store, void* v_store,
                  const int64_t* positions, const int32_t* seq_cols, const int32_t* slot_rows,
                  int T, int Hkv, int D, int rows, int cols, const int64_t kn_str[3],
                  const int64_t vn_str[3], const int64_t ks_str[4], const int64_t vs_str[4],
                  void* workspace, size_t ws_bytes, void* stream) {
    clear_err();
    if (!k_store || !v_store) return fail(ATTN_ERR_INVALID, "null store pointer");
    if (T > 0 && (!k_new || !v_new || !positions || !seq_cols))
        return fail(ATTN_ERR_INVALID, "null tensor pointer");
    if (!kn_str || !vn_str || !ks_str || !vs_str) return fail(ATTN_ERR_INVALID, "null stride array");
    if (T < 0 || Hkv < 1 || D < 1 || rows < 1 || cols < 1)
        return fail(ATTN_ERR_INVALID, "sizes must satisfy T >= 0 and Hkv, D, rows, cols >= 1");
    if (D % 8 != 0 || D > 1024) return fail(ATTN_ERR_UNSUPPORTED, "head dim %d: a multiple of 8 up to 1024", D);
    int st;
    if ((st = check_layout("k_new", k_new, kn_str, 3))) return st;
    if ((st = check_layout("v_new", v_new, vn_str, 3))) return st;
    if ((st = check_layout("k_store", k_store, ks_str, 4))) return st;
    if ((st = check_layout("v_store", v_store, vs_str, 4))) return st;
    if ((uintptr_t)positions % 8 != 0 || (uintptr_t)seq_cols % 4 != 0 ||
        (uintptr_t)slot_rows % 4 != 0)
        return fail(ATTN_ERR_UNSUPPORTED, "per-token arrays are not naturally aligned");
    const int64_t nsz[3] = {T, Hkv, D}, ssz[4] = {rows, cols, Hkv, D};
    if (!offset_ok(nsz, kn_str, 3) || !offset_ok(nsz, vn_str, 3) || !offset_ok(ssz, ks_str, 4) ||
        !offset_ok(ssz, vs_str, 4))
        return fail(ATTN_ERR_INVALID, "element offsets exceed 2^62");
    const size_t need = attn_kv_write_workspace(T);
    if (!workspace || ws_bytes < need)
        return fail(ATTN_ERR_WORKSPACE, "workspace of %zu bytes needed, %zu given", need,
                    workspace ? ws_bytes : (size_t)0);
    if ((uintptr_t)workspace % 256 != 0)
        return fail(ATTN_ERR_WORKSPACE, "workspace is not 256-byte aligned");
    if (T == 0) return ATTN_OK;
    KVWriteArgs a;
    a.kn = (const u16*)k_new;
    a.vn = (const u16*)v_new;
    a.ks = (u16*)k_store;
    a.vs = (u16*)v_store;
    a.pos = positions;
    a.col = seq_cols;
    a.srows = slot_rows;
    a.err = (int32_t*)workspace;
    a.T = T;
    a.Hkv = Hkv;
    a.D = D;
    a.rows = rows;
    a.cols = cols;
    for (int i = 0; i < 3; ++i) {
        a.kns[i] = kn_str[i];
        a.vns[i] = vn_str[i];
    }
    for (int i = 0; i < 4; ++i) {
        a.kss[i] = ks_str[i];
        a.vss[i] = vs_str[i];
    }
    hipLaunchKernelGGL(kv_write_kernel, dim3((unsigned)kv_write_blocks(T)),
                       dim3(kWriteTokens * kWave), 0, (hipStream_t)stream, a);
    if (hipGetLastError() != hipSuccess) return fail(ATTN_ERR_HIP, "slot-write launch failed");
    return ATTN_OK;
}

int attn_kv_write_read_error(const void* workspace, int T, void* stream, int32_t* err_out) {
    clear_err();
    if (!workspace || !err_out) return fail(ATTN_ERR_INVALID, "null pointer");
    if (T < 0) return fail(ATTN_ERR_INVALID, "negative size");
    *err_out = 0;
    const int n = kv_write_blocks(T);
    if (hipStreamSynchronize((hipStream_t)stream) != hipSuccess)
        return fail(ATTN_ERR_HIP, "stream sync failed");
    if (n == 0) return ATTN_OK;
    std::vector<int32_t> host((size_t)n);
    if (hipMemcpy(host.data(), workspace, sizeof(int32_t) * n, hipMemcpyDeviceToHost) != hipSuccess)
        return fail(ATTN_ERR_HIP, "copy of the error word failed");
    int32_t e = 0;
    for (int v : host) e |= v;
    *err_out = e;
    return ATTN_OK;
}

int attn_timing_begin(void) {
    clear_err();
    g_timing.recycle();
    g_timing.on = true;
    g_timing.clk = nullptr;
    g_timing.dev = -1;
    void* p = nullptr;
    int dev = -1;
    if (hipGetDevice(&dev) != hipSuccess || hipGetSymbolAddress(&p, HIP_SYMBOL(g_clock)) != hipSuccess ||
        hipMemset(p, 0, sizeof(g_clock)) != hipSuccess || hipDeviceSynchronize() != hipSuccess) {
        (void)hipGetLastError();
        return ATTN_OK;  // events still time the kernels; the clock reads as unavailable
    }
    g_timing.dev = dev;
    g_timing.clk = (unsigned long long*)p;
    return ATTN_OK;
}

int attn_timing_end(double* kernel_ms, int* launches) {
    clear_err();
    if (!kernel_ms || !launches) return fail(ATTN_ERR_INVALID, "null output pointer");
    g_timing.on = false;
    double total = 0.0;
    int n = 0;
    int st = ATTN_OK;
    for (auto& m : g_timing.marks) {
        float ms = 0.f;
        if (!m.first || !m.second || hipEventSynchronize(m.second) != hipSuccess ||
            hipEventElapsedTime(&ms, m.first, m.second) != hipSuccess) {
            st = fail(ATTN_ERR_HIP, "a timing event could not be read");
            continue;
        }
        total += ms;
        ++n;
    }
    g_timing.recycle();
    *kernel_ms = total;
    *launches = n;
    return st;
}

int attn_timing_clock(double* mhz, double xcd_mhz[8]) {
    clear_err();
    if (!mhz) return fail(ATTN_ERR_INVALID, "null output pointer");
    *mhz = 0.0;
    if (xcd_mhz)
        for (int i = 0; i < 8; ++i) xcd_mhz[i] = 0.0;
    if (g_timing.on) return fail(ATTN_ERR_INVALID, "timing is still on (call attn_timing_end first)");
    if (!g_timing.clk) return fail(ATTN_ERR_HIP, "no clock sums were recorded");
    int cur = -1;
    if (hipGetDevice(&cur) != hipSuccess || hipSetDevice(g_timing.dev) != hipSuccess)
        return fail(ATTN_ERR_HIP, "could not select the timed device");
    unsigned long long h[16];
    hipError_t e = hipMemcpy(h, g_timing.clk, sizeof h, hipMemcpyDeviceToHost);
    (void)hipSetDevice(cur);
    if (e != hipSuccess) return fail(ATTN_ERR_HIP, "copy of the clock sums failed");
    double cyc = 0.0, ref = 0.0;
    for (int i = 0; i < 8; ++i) {
        cyc += (double)h[2 * i];
        ref += (double)h[2 * i + 1];
        if (xcd_mhz && h[2 * i + 1]) xcd_mhz[i] = 100.0 * (double)h[2 * i] / (double)h[2 * i + 1];
    }
    if (ref <= 0.0) return fail(ATTN_ERR_HIP, "no clock sums were recorded");
    *mhz = 100.0 * cyc / ref;
    return ATTN_OK;
}

int attn_timing_reruns(long long* workgroups, long long* redone) {
    clear_err();
    if (!workgroups || !redone) return fail(ATTN_ERR_INVALID, "null output pointer");
    *workgroups = 0;
    *redone = 0;
    if (g_timing.on) return fail(ATTN_ERR_INVALID, "timing is still on (call attn_timing_end first)");
    if (!g_timing.clk) return fail(ATTN_ERR_HIP, "no clock sums were recorded");
    int cur = -1;
    if (hipGetDevice(&cur) != hipSuccess || hipSetDevice(g_timing.dev) != hipSuccess)
        return fail(ATTN_ERR_HIP, "could not select the timed device");
    unsigned long long h[2];
    hipError_t e = hipMemcpy(h, g_timing.clk + 16, sizeof h, hipMemcpyDeviceToHost);
    (void)hipSetDevice(cur);
    if (e != hipSuccess) return fail(ATTN_ERR_HIP, "copy of the workgroup counts failed");
    *workgroups = (long long)h[0];
    *redone = (long long)h[1];
    return ATTN_OK;
}

}  // extern "C"
