// Block attention of one denoising / verify step on gfx950.
//
// Operation (Fast-dVLM write-up, section 4.1 and 5.3; summary page Fig. 3):
// the D slots of the current block attend to the frozen cache positions
// 0..P-1 and to the block itself, bidirectionally (denoise) or causally
// (verify / AR step).  GQA: the Hq/Hkv query heads sharing one KV head are
// processed together as D * Hq/Hkv "grouped rows" against one K/V stream.
//
// MFMA path (bf16 queries, bf16 or E4M3 K/V, d = 64 or 128).  One workgroup
// owns one (item, KV head, row block, key split).  Each wave owns 32 grouped
// rows and computes
//     S^T = K . Q^T        (v_mfma_f32_32x32x16_bf16, keys x rows)
//     O^T += V^T . P^T     (same instruction, d x rows)
// so that each lane holds one query row: the softmax max is an in-lane
// reduction plus one exchange between the two 32-lane halves.  K rows are
// fed to the first MFMA in a permuted order so that the scores a lane holds
// for each 16-key chunk are consecutive keys; the second MFMA then takes its
// V^T operand from the row-major [key][d] value tile through gfx950's LDS
// transpose loads (two 8-byte loads per lane and MFMA), so values are cached
// in the same [cap][d] layout as keys.  K and V tiles (32 bf16 or 64 E4M3
// keys, 8 KB each at d = 128) stream through four LDS stages with XOR
// swizzles that keep every read phase conflict-free.  E4M3 K/V (the FP8 rung of the Fast-dVLM write-up, section
// 5.4 and Table 4, applied to the cache) are widened to bf16 exactly, right
// after each LDS read, with one fp32 scale per (item, KV head) for K and V.
// The online softmax (Milakov & Gimelshein, "Online normalizer calculation
// for softmax", 2018) only rescales when the running maximum grows by more
// than 2^8, which keeps every exponent <= 2^8 and is exact after the final
// normalisation.  The cached prefix is split across workgroups (split-K);
// a second kernel merges each unit's (m, l, o) partials in split order, so
// results do not depend on scheduling.
#include <type_traits>

#include "bd_common.h"
#include "bd_internal.h"

namespace bd {
namespace {

struct MfmaParams {
    const uint16_t *q;
    const uint8_t *kb, *vb, *kc, *vc;  // K / V storage (bf16 or E4M3), byte addressed
    const int32_t *prefix;
    const float *k_scale, *v_scale;    // [n][Hkv], E4M3 K / V only
    uint16_t *out;
    float *ws_o;
    float2 *ws_ml;
    int n, D, Hq, Hkv, G, cap, mode;
    int B;  // quadratic mode: draft block size (D = B (B + 3) / 2 slots)
    int R, row_blocks, max_splits, tiles_per_split, total_logical;
    int balanced;       // ragged-batch plan: split counts from the device-side prefix lengths
    int balance_slots;  // ... workgroups the plan may use
    float c;  // scale * log2(e)
    // Two-stream (whole-sequence) mode: D = L = Lc + Ln positions per item, the
    // clean stream then the noisy stream; response spans (clean start, length).
    const int32_t *spans, *n_spans;
    int *unit_splits;  // [units]: split count of each unit, for the merge kernel
    int Lc, max_spans, Dblk;
    int max_prefix;  // the host's longest prefix (<= cap): paired halves plan their first copies with it
};

// Block slots a query slot may attend to, as two half-open slot ranges
// [0, hi1) and [lo2, hi2).  Cache positions, given as negative slot numbers,
// are visible to every slot (hi1 >= 0).
//  BIDIR (mode 0): the whole block.  CAUSAL (mode 1): slots 0..slot.
//  QUAD (mode 2), the quadratic self-speculative block (Fast-dVLM write-up,
//  section 5.3): slots 0..B-1 are the drafts, causal among themselves; then
//  group g = 0..B-1 holds B - g mask tokens, which see drafts 0..g-1 and
//  every mask token of their own group.
struct SlotRanges {
    int hi1, lo2, hi2;
};
__device__ __forceinline__ SlotRanges block_ranges(int mode, int slot, int D, int B) {
    if (mode == 0) return {D, 0, 0};
    if (mode == 1 || slot < B) return {slot + 1, 0, 0};
    int m = slot - B, g = 0, start = B;
    while (g < B && m >= B - g) {
        m -= B - g;
        start += B - g;
        ++g;
    }
    return {g, start, start + (B - g)};
}
// Bitwise, not short-circuit: the result feeds a select, with no branches.
__device__ __forceinline__ bool in_ranges(const SlotRanges &r, int b) {
    return (b < r.hi1) | ((b >= r.lo2) & (b < r.hi2));
}

// Two-stream training attention (Fast-dVLM write-up, sections 4.1, 4.3, 4.4;
// summary page Fig. 3): the keys a sequence position sees, as key-position
// ranges [0, hi1) and [lo2, hi2) of [clean stream ; noisy stream].
//  clean position p          : clean keys 0..p (token causal);
//  noisy position Lc + i     : i falls in response r (noisy offset o, clean
//                              start c, length len), block k = (i - o) / Dblk;
//                              clean keys before c + k Dblk, and the noisy keys
//                              of its block, cut at the response end;
//  noisy positions past the last response see nothing.
// Spans come from device memory: every bound is clamped into the sequence.
__device__ __forceinline__ SlotRanges seq_ranges(const MfmaParams &p, int it, int pos) {
    if (pos < p.Lc) return {pos + 1, 0, 0};
    const int L = p.D;
    const int i = pos - p.Lc;
    const int32_t *sp = p.spans + (size_t)it * p.max_spans * 2;
    const int ns = min(max(p.n_spans[it], 0), p.max_spans);
    int o = 0;
    for (int r = 0; r < ns; ++r) {
        const int c = sp[2 * r], len = max(sp[2 * r + 1], 0);
        if (i < o + len) {
            const int k = (i - o) / p.Dblk;
            const int b0 = min(max(c + k * p.Dblk, 0), p.Lc);
            const int w0 = o + k * p.Dblk;
            const int bl = min(p.Dblk, len - k * p.Dblk);
            return {b0, min(p.Lc + w0, L), min(p.Lc + w0 + bl, L)};
        }
        o += len;
    }
    return {0, 0, 0};
}

// A workgroup-uniform pointer, moved into scalar registers (an operand of a
// scalar load written in inline assembly must be one).
__device__ __forceinline__ const int32_t *bd_uniform_ptr(const int32_t *q) {
    const uint64_t v = (uint64_t)q;
    const uint32_t lo = (uint32_t)__builtin_amdgcn_readfirstlane((int)(uint32_t)v);
    const uint32_t hi = (uint32_t)__builtin_amdgcn_readfirstlane((int)(uint32_t)(v >> 32));
    return (const int32_t *)(((uint64_t)hi << 32) | lo);
}

// Paired halves: the plan of one list slot (see attn_mfma_kernel).
struct SlotPlan {
    bool valid;
    int unit, nsplit, t0, nb, ntail;
};

// Row permutations of the K operand.  A-row rho (= lane % 32) of a 32-key
// block loads key pi(rho).
//  bf16: output register i of half h then holds key 16 (i / 8) + 8 h + (i % 8),
//        so 16-key chunk c of the second product is registers 8 (c % 2) .. of
//        block c / 2 and its V^T operand is one 16-byte unit (8 keys) per lane.
//  E4M3: register i of half h holds key 16 h + i.  Chunk c = 2m + j then
//        covers keys 32m + 16h + 8j .. +7 for half h, which are bytes
//        8j .. 8j+7 of the 16-byte unit 2m + h of a V^T row: one LDS read
//        feeds the operands of two chunks.
__device__ __forceinline__ int key_perm(int rho) {
    int q = rho >> 3, h = (rho >> 2) & 1, e = rho & 3;
    return ((q >> 1) << 4) + (h << 3) + ((q & 1) << 2) + e;
}
__device__ __forceinline__ int key_perm8(int rho) {
    return (((rho >> 2) & 1) << 4) + ((rho >> 3) << 2) + (rho & 3);
}

// Work split of a unit with prefix P and TK-key tiles.  The unit streams
// nbulk = P / TK whole cache tiles plus ntail tail tiles (the last P % TK
// cache positions and the D block slots, gathered by a slower path that costs
// about kTailCost bulk tiles).  nsplit = ceil(work / tiles_per_split) splits,
// at most max_splits and at most nbulk + 1; the last split runs the tail and
// takes whatever bulk tiles are left once the others have ceil(work / nsplit)
// each, so that no split carries much more than the average.  Shared by the
// tile and merge kernels.
constexpr int kTailCost = 3;
struct UnitSplit {
    int nsplit;  // splits of this unit (the last one holds the tail)
    int t0, nb;  // bulk tile range of the queried split
};
template <int TK>
__device__ __forceinline__ int unit_nsplit(int P, int D, int tiles_per_split, int max_splits) {
    const int nbulk = P / TK;
    const int ntail = ((P - nbulk * TK) + D + TK - 1) / TK;
    const int work = nbulk + kTailCost * ntail;
    return max(1, min(min(max_splits, nbulk + 1), (work + tiles_per_split - 1) / tiles_per_split));
}
// The split of a unit with `nsplit` splits (1 <= nsplit <= nbulk + 1).
template <int TK>
__device__ __forceinline__ UnitSplit unit_split_n(int P, int D, int nsplit, int split) {
    UnitSplit u;
    const int nbulk = P / TK;
    const int ntail = ((P - nbulk * TK) + D + TK - 1) / TK;
    const int work = nbulk + kTailCost * ntail;
    u.nsplit = nsplit;
    const int nbs = u.nsplit - 1;                                      // bulk-only splits
    const int w = (work + u.nsplit - 1) / u.nsplit;                    // target work per split
    const int tail_bulk = nbs == 0 ? nbulk : max(0, nbulk - nbs * w);  // bulk tiles of the tail split
    const int shared = nbulk - tail_bulk;                              // >= nbs: every bulk split gets one
    // 32-bit arithmetic is enough: split < kMaxSplits = 64 and shared <= cap / TK < 2^19.
    if (split < nbs) {
        u.t0 = (int)((unsigned)(split * shared) / (unsigned)nbs);
        u.nb = (int)((unsigned)((split + 1) * shared) / (unsigned)nbs) - u.t0;
    } else {
        u.t0 = shared;
        u.nb = tail_bulk;
    }
    return u;
}
template <int TK>
__device__ __forceinline__ UnitSplit unit_split(int P, int D, int tiles_per_split, int max_splits, int split) {
    return unit_split_n<TK>(P, D, unit_nsplit<TK>(P, D, tiles_per_split, max_splits), split);
}

// Sum and max over the 64 lanes of a wave with DPP row operations and lane
// swaps (no LDS round trip); every lane receives the result.
template <int CTRL>
__device__ __forceinline__ int dpp_i(int x) { return __builtin_amdgcn_update_dpp(0, x, CTRL, 0xf, 0xf, false); }
__device__ __forceinline__ int wave_sum_i(int x) {
    x += dpp_i<0xB1>(x);
    x += dpp_i<0x4E>(x);
    x += dpp_i<0x141>(x);
    x += dpp_i<0x140>(x);
    const auto a = __builtin_amdgcn_permlane16_swap((unsigned)x, (unsigned)x, false, false);
    x = (int)(a[0] + a[1]);
    const auto b = __builtin_amdgcn_permlane32_swap((unsigned)x, (unsigned)x, false, false);
    return (int)(b[0] + b[1]);
}
__device__ __forceinline__ int wave_max_i(int x) {
    x = max(x, dpp_i<0xB1>(x));
    x = max(x, dpp_i<0x4E>(x));
    x = max(x, dpp_i<0x141>(x));
    x = max(x, dpp_i<0x140>(x));
    const auto a = __builtin_amdgcn_permlane16_swap((unsigned)x, (unsigned)x, false, false);
    x = max((int)a[0], (int)a[1]);
    const auto b = __builtin_amdgcn_permlane32_swap((unsigned)x, (unsigned)x, false, false);
    return max((int)b[0], (int)b[1]);
}

// Split plan of a ragged batch (items with different prefix lengths, at most
// 64 of them: one lane per item).  Every unit of item i gets
//   n_i = min(cap_i, ceil(work_i / T)) splits,   cap_i = min(max_splits, nbulk_i + 1),
// with T the smallest whole number of tiles for which the splits of all units
// fit `balance_slots` workgroups, so the longest split of the call is as short
// as that many workgroups allow (a plan sized from the host's max_prefix gives
// short items few splits and leaves CUs idle).  It depends only on the
// prefix lengths, so every wave that computes it gets the same plan and the
// results do not depend on scheduling.  Lane i returns n_i and the first
// logical workgroup of item i's units (unit-major: units of item i, in order,
// n_i splits each); `total` is the workgroup count.
struct ItemPlan {
    int nsplit, start, total;
    int prefix;  // lane i: item i's prefix length (clamped into [0, cap])
};
template <int TK>
__device__ __forceinline__ ItemPlan balanced_plan(const MfmaParams &p, int lane) {
    const bool has = lane < p.n;
    const int P = has ? min(max(p.prefix[lane], 0), p.cap) : 0;
    const int nbulk = P / TK;
    const int ntail = ((P - nbulk * TK) + p.D + TK - 1) / TK;
    const int work = has ? nbulk + kTailCost * ntail : 0;
    const int capi = min(p.max_splits, nbulk + 1);
    const int upi = p.Hkv * p.row_blocks;  // units per item
    // count(T) = upi * sum_i min(cap_i, ceil(work_i / T)) falls as T grows; at
    // T = max work it is the unit count, which the host keeps <= balance_slots.
    int lo = 1, hi = max(1, wave_max_i(work));
    while (lo < hi) {
        const int mid = (lo + hi) >> 1;
        const int c = has ? min(capi, (work + mid - 1) / mid) : 0;
        if (wave_sum_i(c) * upi <= p.balance_slots)
            hi = mid;
        else
            lo = mid + 1;
    }
    ItemPlan ip;
    ip.nsplit = has ? min(capi, (work + lo - 1) / lo) : 0;
    ip.prefix = P;
    const int cnt = ip.nsplit * upi;
    int incl = cnt;  // inclusive prefix sum over the lanes
#pragma unroll
    for (int off = 1; off < 64; off <<= 1) {
        const int v = __shfl_up(incl, off, 64);
        if (lane >= off) incl += v;
    }
    ip.start = incl - cnt;
    ip.total = __shfl(incl, 63, 64);
    return ip;
}

// 16-byte-unit XOR swizzles of the LDS tiles.  A tile row of U units shares
// one 256-byte bank span (16 units) with 16/U - 1 other rows.  One ds_read_b128
// phase serves 16 lanes that read the same logical unit of 16 different rows;
// the swizzle sends those 16 reads to 16 different unit slots of the span.
// bf16 K rows are read 16 consecutive rows at a time.
template <int U>
__device__ __forceinline__ int row_swz(int row) { return (row / (16 / U)) & (U - 1); }
// E4M3 K rows are read in key_perm8 order: the 16 keys of a phase differ in
// bits 0-2 and 4 (bit 3 fixed), so the swizzle is taken from those bits.
template <int HD, bool KV8>
__device__ __forceinline__ int k_swz(int key) {
    if constexpr (!KV8) return row_swz<HD / 8>(key);
    else if constexpr (HD == 128) return ((key >> 1) & 3) | ((key >> 2) & 4);  // 2 rows per span
    else return ((key >> 2) & 1) | ((key >> 3) & 2);                             // 4 rows per span
}
// V rows ([key][d], U units each) are read by LDS transpose loads: in every
// 32-lane phase, bf16 reads cover 4 consecutive rows x 64 bytes and E4M3 reads
// 8 consecutive rows x 32 bytes.  The swizzle moves the 64- (32-) byte column
// chunk of each of those rows to its own quarter (eighth) of the 256-byte bank
// span.  It depends on key mod 4 (bf16) or key mod 8 (E4M3) only.
template <int HD, bool KV8>
__device__ __forceinline__ int v_swz(int key) {
    constexpr int U = HD * (KV8 ? 1 : 2) / 16;  // 16-byte units per row
    constexpr int RPS = 16 / U;                 // rows per 256-byte span
    if constexpr (!KV8) return 4 * ((key / RPS) % (U / 4));
    else return 2 * ((key / RPS) % (U / 2));
}

// LDS transpose loads of gfx950.  In each group of 16 lanes every lane fetches
// 8 bytes at its own address; ds_read_b64_tr_b16 then gives lane r, element j
// (0..3) the 16-bit element r % 4 of lane 4 j + r / 4's fetch, and
// ds_read_b64_tr_b8 gives lane r, byte j (0..7) the byte r % 8 of lane
// 2 j + r / 8's fetch.  So when the 16 lanes fetch 4 (8) consecutive rows of a
// row-major [key][d] tile, 4 (2) lanes per row over 16 consecutive columns,
// lane r receives column r of those 4 (8) rows: the k-contiguous operand an
// MFMA takes.
typedef short bd_s16x4 __attribute__((ext_vector_type(4)));
typedef int bd_i32x2 __attribute__((ext_vector_type(2)));
__device__ __forceinline__ bd_s16x4 bd_lds_tr16(const uint8_t *p) {
    return __builtin_amdgcn_ds_read_tr16_b64_v4i16(
        (__attribute__((address_space(3))) bd_s16x4 *)(__attribute__((address_space(3))) uint8_t *)p);
}
__device__ __forceinline__ bd_i32x2 bd_lds_tr8(const uint8_t *p) {
    return __builtin_amdgcn_ds_read_tr8_b64_v2i32(
        (__attribute__((address_space(3))) bd_i32x2 *)(__attribute__((address_space(3))) uint8_t *)p);
}

// Tile pipeline depth: NS LDS stages per workgroup, so NS - 1 tiles stay in
// flight while one is computed.  A stage holds 32 bf16 keys or 64 E4M3 keys:
// with d = 128, four stages take 64 KB of LDS and two workgroups (two waves
// per SIMD) share a CU, each keeping three tiles (48 KB) in flight.  Two per
// CU is also the cap for d = 64, where registers rather than LDS are the limit.
constexpr int kStages = 4;
#ifndef BD_PAIR_HALVES
#define BD_PAIR_HALVES 1
#endif
constexpr int kStageBytesPerD = kTileKeys * 2;  // LDS bytes of one K (or V) stage per head-dim element
constexpr int occupancy_for(int hd) {
    return (160 * 1024) / (kStages * 2 * kStageBytesPerD * hd) < 2 ? (160 * 1024) / (kStages * 2 * kStageBytesPerD * hd)
                                                                   : 2;
}

// Two E4M3 values (bytes 2 SEL, 2 SEL + 1 of w) -> two bf16, exact (every
// E4M3 value is a bf16 value), with v_cvt_scalef32_pk_bf16_fp8 at scale 1.
template <bool SEL>
__device__ __forceinline__ bf16x2 bd_e4m3x2_to_bf16(uint32_t w) {
    return __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w, 1.0f, SEL);
}
// Eight E4M3 bytes (lo, hi) -> one bf16x8 MFMA operand, byte order kept.
__device__ __forceinline__ bf16x8 bd_e4m3x8_to_bf16(uint32_t lo, uint32_t hi) {
    const bf16x2 a = bd_e4m3x2_to_bf16<false>(lo), b = bd_e4m3x2_to_bf16<true>(lo);
    const bf16x2 c = bd_e4m3x2_to_bf16<false>(hi), d = bd_e4m3x2_to_bf16<true>(hi);
    return bf16x8{a[0], a[1], b[0], b[1], c[0], c[1], d[0], d[1]};
}

// KV8 = false: bf16 K / V, 32-key tiles.  KV8 = true: E4M3 K / V with one
// fp32 scale per (item, KV head) for K and for V, 64-key tiles (the same
// bytes per stage), converted to bf16 right after each LDS read; the K scale
// is folded into the softmax constant and the V scale into the final
// normalisation.
// SEQ = true: two-stream training attention over whole sequences (bf16 K/V):
// every key tile comes from the item's K/V arrays by the same copy pipeline,
// and tiles that some row of the workgroup only partly sees are masked.
// PAIR = true (block modes, d = 128): one workgroup per CU of two NW-wave
// halves.  Half h runs split slot 2 L + h of the call's unit-major slot list
// (L = the workgroup's logical id) with its own four LDS stages; both halves
// step through one barrier sequence, sized for the longer of the two, so
// they keep pace instead of the later-dispatched of two workgroups on a CU
// falling behind.  When both slots belong to one unit (same rows, adjacent
// key ranges), the halves combine their (m, l, o) through LDS and the pair
// leaves one partial; the merge kernel skips the slot it absorbed.
template <int HD, int NW, bool KV8, bool SEQ, bool PAIR = false>
__global__ __launch_bounds__(NW * 64 * (PAIR ? 2 : 1), occupancy_for(HD)) void attn_mfma_kernel(MfmaParams p) {
    static_assert(!(SEQ && KV8), "the sequence mode is bf16 only");
    static_assert(!(SEQ && PAIR) && (!PAIR || HD == 128), "paired halves: block modes, d = 128");
    constexpr int NH = PAIR ? 2 : 1;    // halves per workgroup
    constexpr int NT = NW * 64;         // threads per half
    constexpr int EB = KV8 ? 1 : 2;     // bytes per K / V element
    constexpr int TK = KV8 ? 2 * kTileKeys : kTileKeys;  // keys per tile
    constexpr int KU = HD * EB / 16;    // 16-byte units per K (or V) row
    constexpr int SB = TK * HD * EB;    // bytes per K (or V) stage
    constexpr int K_UNITS = TK * KU;    // ... and V units: both tiles are [TK][HD]
    constexpr int LK = (K_UNITS + NT - 1) / NT;
    constexpr int LV = LK;
    constexpr int KC = HD / 16;         // d-chunks of the first MFMA
    constexpr int MB = HD / 32;         // d-blocks of the second MFMA
    constexpr int RPG = NW * 32;        // rows per workgroup
    constexpr int KB = TK / 32;         // 32-key blocks of the first MFMA per tile
    constexpr int C4 = TK / 16;         // 16-key chunks of the second MFMA per tile
    constexpr int NS = kStages;
    static_assert(SB == kStageBytesPerD * HD, "stage size must match occupancy_for");
    static_assert(NS == 4, "the stage arrays below are written out for four stages");
    static_assert((NS - 1) * (LK + LV) < 64, "outstanding copies must fit the vmcnt counter");

    // One array per stage: the tile loop below is unrolled by NS so that every
    // LDS access names a fixed array, which lets the compiler see that reads of
    // one stage never alias the global->LDS copies in flight into the others.
    // With paired halves each array holds one stage of each half.
    __shared__ __attribute__((aligned(16))) uint8_t lds_k0[SB * NH];
    __shared__ __attribute__((aligned(16))) uint8_t lds_k1[SB * NH];
    __shared__ __attribute__((aligned(16))) uint8_t lds_k2[SB * NH];
    __shared__ __attribute__((aligned(16))) uint8_t lds_k3[SB * NH];
    __shared__ __attribute__((aligned(16))) uint8_t lds_v0[SB * NH];
    __shared__ __attribute__((aligned(16))) uint8_t lds_v1[SB * NH];
    __shared__ __attribute__((aligned(16))) uint8_t lds_v2[SB * NH];
    __shared__ __attribute__((aligned(16))) uint8_t lds_v3[SB * NH];
    // This thread's half and its index within the half.
    const int hw = PAIR ? __builtin_amdgcn_readfirstlane((int)threadIdx.x / NT) : 0;  // wave-uniform
    const int tid = (int)threadIdx.x - hw * NT;
    const int hoff = hw * SB;
    auto kraw = [&](int st) __attribute__((always_inline)) -> uint8_t * {
        return st == 0 ? lds_k0 : st == 1 ? lds_k1 : st == 2 ? lds_k2 : lds_k3;
    };
    auto vraw = [&](int st) __attribute__((always_inline)) -> uint8_t * {
        return st == 0 ? lds_v0 : st == 1 ? lds_v1 : st == 2 ? lds_v2 : lds_v3;
    };
    auto kbuf = [&](int st) __attribute__((always_inline)) -> uint8_t * { return kraw(st) + hoff; };
    auto vbuf = [&](int st) __attribute__((always_inline)) -> uint8_t * { return vraw(st) + hoff; };
    // Byte offsets of 16-byte unit lu of K / V row `key` in a stage.
    auto k_at = [](int key, int lu) __attribute__((always_inline)) { return (key * KU + (lu ^ k_swz<HD, KV8>(key))) * 16; };
    auto v_at = [](int key, int lu) __attribute__((always_inline)) { return (key * KU + (lu ^ v_swz<HD, KV8>(key))) * 16; };

    const int lane = tid & 63;
    const int w = tid >> 6;
    const int half = lane >> 5;
    const int col = lane & 31;

    // XCD-aware decode: consecutive logical ids (the splits of one unit) share an XCD.
    const int nb = gridDim.x;
    const int logical = (blockIdx.x & 7) * (nb >> 3) + (blockIdx.x >> 3);
    int unit, split, nsplit_b = 0;  // nsplit_b: the balanced plan's split count of this unit
    int pre0 = 0, pre1 = 0;  // paired halves: the prefix lengths of slots 2 L and 2 L + 1
    if constexpr (!SEQ && !KV8) {
        // Every kernel argument the prologue uses, fetched in one batch at
        // entry rather than in several dependent round trips (not for E4M3,
        // where the registers it keeps live would spill).
        asm volatile("" ::"s"(p.total_logical), "s"(p.max_splits), "s"(p.row_blocks), "s"(p.Hkv), "s"(p.G),
                     "s"(p.R), "s"(p.D), "s"(p.Hq), "s"(p.q), "s"(p.prefix), "s"(p.cap), "s"(p.tiles_per_split),
                     "s"(p.mode), "s"(p.B), "s"(p.kc), "s"(p.vc), "s"(p.kb), "s"(p.vb), "s"(p.c), "s"(p.balanced),
                     "s"(p.max_prefix));
    }
    if (PAIR) {
        // Slot 2 L + hw of the list; a half past its end takes its partner's
        // unit for the addresses below and streams nothing.
        if (2 * logical >= p.total_logical) return;  // both halves: the whole workgroup
        const int sidx = min(2 * logical + hw, p.total_logical - 1);
        unit = sidx / p.max_splits;
        split = sidx - unit * p.max_splits;
    } else if (!SEQ && p.balanced) {
        const ItemPlan ip = balanced_plan<TK>(p, lane);
        if (logical >= ip.total) return;  // the whole workgroup: every wave has the same plan
        const int upi = p.Hkv * p.row_blocks;
        const unsigned long long hit =
            __builtin_amdgcn_ballot_w64(lane < p.n && logical >= ip.start && logical < ip.start + ip.nsplit * upi);
        const int item = __builtin_ctzll(hit);
        nsplit_b = __shfl(ip.nsplit, item, 64);
        pre0 = __shfl(ip.prefix, item, 64);
        const int rloc = logical - __shfl(ip.start, item, 64);
        const int uin = rloc / nsplit_b;
        split = rloc - uin * nsplit_b;
        unit = item * upi + uin;
        // The merge kernel reads the count here instead of recomputing the plan.
        if (split == 0 && tid == 0) p.unit_splits[unit] = nsplit_b;
    } else {
        if (logical >= p.total_logical) return;
        unit = logical / p.max_splits;
        split = logical - unit * p.max_splits;
    }
    const int rb = unit % p.row_blocks;
    const int pair = unit / p.row_blocks;
    const int g = pair % p.Hkv;
    const int it = pair / p.Hkv;

    // This lane's query row.  Its loads are issued before the prefix length
    // is known (they do not depend on it), so the two round trips overlap.
    // MFMA kc reads d = 16 kc + 8 half .. +7 (bf16) or, in the order an
    // E4M3 K unit is split into two operands, d = 32 (kc/2) + 16 half + 8 (kc%2) .. +7.
    const int r_local = w * 32 + col;
    const int r = rb * RPG + r_local;
    const bool row_valid = r < p.R;
    const bool wave_active = rb * RPG + w * 32 < p.R;
    const int slot = r / p.G;
    const int head = g * p.G + (r - slot * p.G);
    SlotRanges vis{0, 0, 0};
    if (row_valid) vis = SEQ ? seq_ranges(p, it, slot) : block_ranges(p.mode, slot, p.D, p.B);
    bf16x8 qf[KC];
    {
        const uint16_t *qp = p.q + (((size_t)it * p.D + slot) * p.Hq + head) * HD;
#pragma unroll
        for (int kc = 0; kc < KC; ++kc) {
            const int d0 = KV8 ? (kc >> 1) * 32 + half * 16 + (kc & 1) * 8 : kc * 16 + half * 8;
            if (row_valid)
                qf[kc] = *reinterpret_cast<const bf16x8 *>(qp + d0);
            else
                qf[kc] = bf16x8{};
        }
    }
    // Sequence mode: the workgroup's key tiles are segment A, tiles 0..nA-1 of
    // the clean stream (the first nU of them seen whole by every row), then
    // segment B, the noisy tiles from bB on; each row's ranges decide the rest.
    int nU = 0, nA = 0, bB = 0;
    // Key tile of list entry k (sequence mode) or bulk tile k.
    auto tile_of = [&](int k) __attribute__((always_inline)) { return SEQ && k >= nA ? bB + (k - nA) : k; };

    // Byte offset of this (item, KV head)'s K and V cache rows ([cap][HD] each).
    const size_t kc_base = ((size_t)it * p.Hkv + g) * p.cap * HD * EB;

    // Bulk tiles are copied global -> LDS by the load units directly
    // (global_load_lds_dwordx4): each instruction fills 64 consecutive 16-byte
    // LDS slots, one per lane, so the XOR swizzle is applied by choosing every
    // lane's source address.  No VGPRs hold tile data.
    static_assert(K_UNITS % NT == 0, "tile units must split evenly over lanes");
    auto issue_bulk = [&](int t, int st, bool real) __attribute__((always_inline)) {
        const int key0 = tile_of(t) * TK;
#pragma unroll
        for (int j = 0; j < LK; ++j) {
            const int base = (j * NW + w) * 64;
            const int u = base + lane;
            const int key = u / KU, pu = u % KU;
            const int lu = pu ^ k_swz<HD, KV8>(key);
            const uint8_t *src = real ? p.kc + kc_base + (size_t)(key0 + key) * HD * EB + lu * 16 : p.kc + kc_base;
            __builtin_amdgcn_global_load_lds(src, (lds_ptr_t)&kbuf(st)[base * 16], 16, 0, 0);
        }
#pragma unroll
        for (int j = 0; j < LV; ++j) {
            const int base = (j * NW + w) * 64;
            const int u = base + lane;
            const int key = u / KU, pu = u % KU;
            const int lu = pu ^ v_swz<HD, KV8>(key);
            const uint8_t *src = real ? p.vc + kc_base + (size_t)(key0 + key) * HD * EB + lu * 16 : p.kc + kc_base;
            __builtin_amdgcn_global_load_lds(src, (lds_ptr_t)&vbuf(st)[base * 16], 16, 0, 0);
        }
    };
    // Paired halves: the plan of list slot s for a prefix length.  The slots
    // of an odd unit take its key ranges in reverse (slot s runs split
    // nsplit - 1 - s), so with an odd slot count per unit the two tail splits
    // of units 2k and 2k + 1 share a workgroup, which then steps through fewer
    // bulk tiles, instead of each tail holding up a partner with a full share.
    auto slot_plan = [&](int s, int raw_prefix) __attribute__((always_inline)) {
        SlotPlan sp{false, -1, 1, 0, 0, 0};
        if (s >= p.total_logical) return sp;
        sp.unit = s / p.max_splits;
        const int sl = s - sp.unit * p.max_splits;
        const int Px = min(max(raw_prefix, 0), p.cap);
        sp.nsplit = unit_nsplit<TK>(Px, p.D, p.tiles_per_split, p.max_splits);
        if (sl >= sp.nsplit) return sp;
        const int kx = (sp.unit & 1) ? sp.nsplit - 1 - sl : sl;
        const UnitSplit u = unit_split_n<TK>(Px, p.D, sp.nsplit, kx);
        sp.valid = true;
        sp.t0 = u.t0;
        sp.nb = u.nb;
        sp.ntail = kx == sp.nsplit - 1 ? ((Px - (Px & ~(TK - 1))) + p.D + TK - 1) / TK : 0;
        return sp;
    };
    // Paired halves: a half whose slot, planned with the host's max_prefix,
    // streams bulk tiles only issues that plan's first NS - 1 tile copies now,
    // before its prefix length is known (for a batch of equal prefixes the
    // plan is exact); if the real plan differs, the half drains these copies
    // and issues its own (below).  Not for E4M3 caches, where the extra live
    // registers cost more than the earlier start gains.
    bool spec = false;
    int spec_t0 = 0, spec_nb = 0;
    if constexpr (PAIR && !KV8) {
        const SlotPlan sp = slot_plan(2 * logical + hw, p.max_prefix);
        spec = sp.valid && sp.ntail == 0 && sp.nb > 0;
        spec_t0 = sp.t0;
        spec_nb = sp.nb;
        if (spec) {
#pragma unroll
            for (int i = 0; i < NS - 1; ++i) issue_bulk(spec_t0 + i, i, i < spec_nb);
        }
    }
    // The prefix lengths this workgroup plans with (workgroup-uniform
    // addresses) as scalar loads issued after the query loads and waited for
    // on the scalar counter alone, so their round trip overlaps the query
    // loads rather than following them (a vector load's wait would also wait
    // for the queries).  Paired halves: slots 2 L and 2 L + 1; otherwise the
    // item's own (the balanced plan has already read every item's).
    if constexpr (PAIR) {
        const int32_t *a0 = bd_uniform_ptr(p.prefix + (2 * logical) / p.max_splits / p.row_blocks / p.Hkv);
        const int32_t *a1 =
            bd_uniform_ptr(p.prefix + min(2 * logical + 1, p.total_logical - 1) / p.max_splits / p.row_blocks / p.Hkv);
        // Early-clobber outputs: the first load's destination must not share a
        // register with the second load's address.
        asm volatile("s_load_dword %0, %2, 0x0\n\ts_load_dword %1, %3, 0x0\n\ts_waitcnt lgkmcnt(0)"
                     : "=&s"(pre0), "=&s"(pre1)
                     : "s"(a0), "s"(a1)
                     : "memory");
    } else if constexpr (!SEQ) {
        if (!p.balanced) {
            const int32_t *a0 = bd_uniform_ptr(p.prefix + it);
            asm volatile("s_load_dword %0, %1, 0x0\n\ts_waitcnt lgkmcnt(0)" : "=&s"(pre0) : "s"(a0) : "memory");
        }
    }
    // Transpose-load offsets of this lane in a V stage, per 32-column block mb.
    // In its group of 16 lanes (s = lane % 16), lane s fetches 8 bytes of row
    // rho = 8 half + s / 4 (bf16) or 16 half + s / 2 (E4M3) at column
    // 32 mb + 16 grp + 4 (s % 4) (bf16) or + 8 (s % 2) (E4M3), grp = lane / 16 % 2;
    // the tile's other rows for this lane are rho plus multiples of 4 (8), which
    // v_swz maps the same way.
    int v_lane[MB];
    {
        const int s16 = lane & 15, grp = (lane >> 4) & 1;
        const int rho = KV8 ? 16 * half + (s16 >> 1) : 8 * half + (s16 >> 2);
        const int cbyte = KV8 ? 16 * grp + 8 * (s16 & 1) : (16 * grp + 4 * (s16 & 3)) * 2;
#pragma unroll
        for (int mb = 0; mb < MB; ++mb) {
            const int c = mb * 32 * EB + cbyte;  // byte column in the row
            v_lane[mb] = v_at(rho, c >> 4) + (c & 15);
        }
    }
    float cs = p.c, vs = 1.0f;
    if constexpr (KV8) {
        cs *= p.k_scale[it * p.Hkv + g];
        vs = p.v_scale[it * p.Hkv + g];
    }

    // Prefix lengths are clamped into [0, cap] so that no access leaves the cache.
    const int P = SEQ ? 0 : min(max(PAIR && hw ? pre1 : pre0, 0), p.cap);
    const int Pb = P & ~(TK - 1);  // cache positions in whole tiles
    int nsplit = 1, t0 = 0, nb_split = 0, tail_len = 0, ntail = 0;
    if constexpr (SEQ) {
        __shared__ int red[4];
        if (tid == 0) {
            red[0] = 0x7fffffff;
            red[1] = 0;
            red[2] = 0x7fffffff;
            red[3] = 0;
        }
        bd_barrier_lds();
        {
            // Each wave reduces its rows' bounds first (rows that see no
            // second range, and invalid rows, contribute the identities), so
            // the workgroup's four LDS atomics are one per wave.
            const bool two = row_valid && vis.hi2 > vis.lo2;
            const int mn0 = wave_max_i(-(row_valid ? vis.hi1 : 0x7fffffff));
            const int mx1 = wave_max_i(row_valid ? vis.hi1 : 0);
            const int mn2 = wave_max_i(-(two ? vis.lo2 : 0x7fffffff));
            const int mx3 = wave_max_i(two ? vis.hi2 : 0);
            if (lane == 0) {
                atomicMin(&red[0], -mn0);
                atomicMax(&red[1], mx1);
                atomicMin(&red[2], -mn2);
                atomicMax(&red[3], mx3);
            }
        }
        bd_barrier_lds();
        const int min_hi1 = red[0], max_hi1 = red[1], min_lo2 = red[2], max_hi2 = red[3];
        nU = min_hi1 == 0x7fffffff ? 0 : min_hi1 / TK;
        nA = (max_hi1 + TK - 1) / TK;
        int nB = 0;
        if (max_hi2 > min_lo2) {
            bB = max(min_lo2 / TK, nA);
            nB = max(0, (max_hi2 + TK - 1) / TK - bB);
        }
        const int nt = nA + nB;
        nsplit = nt == 0 ? 1 : max(1, min(min(p.max_splits, nt), (nt + p.tiles_per_split - 1) / p.tiles_per_split));
        if (split == 0 && tid == 0 && p.unit_splits) p.unit_splits[unit] = nsplit;
        if (split >= nsplit) return;
        t0 = (int)((unsigned)(split * nt) / (unsigned)nsplit);
        nb_split = (int)((unsigned)((split + 1) * nt) / (unsigned)nsplit) - t0;
    } else if constexpr (!PAIR) {
        // A prefix above the host's max_prefix widens the splits instead of
        // overrunning the workspace (at most max_splits per unit).
        const UnitSplit us = p.balanced ? unit_split_n<TK>(P, p.D, nsplit_b, split)
                                        : unit_split<TK>(P, p.D, p.tiles_per_split, p.max_splits, split);
        nsplit = us.nsplit;
        if (split >= nsplit) return;
        const bool is_tail = split == nsplit - 1;
        t0 = us.t0;
        nb_split = us.nb;
        tail_len = is_tail ? (P - Pb) + p.D : 0;
        ntail = is_tail ? (tail_len + TK - 1) / TK : 0;
    }
    // Paired halves: both halves' plans, computed alike by every wave from the
    // list slots and their prefix lengths alone, so the loop counts below (the
    // longer half's tail and bulk tile counts) and every branch around a
    // barrier are the same in all eight waves; each half takes its own.
    bool hvalid = true, merged = false;
    int ntail_all = ntail, nb_all = nb_split;
    if constexpr (PAIR) {
        const SlotPlan s0 = slot_plan(2 * logical, pre0), s1 = slot_plan(2 * logical + 1, pre1);
        if (!s0.valid && !s1.valid) {  // the whole workgroup
            if (spec) bd_wait_vmcnt<0>();  // no copy into this workgroup's LDS outlives it
            return;
        }
        const SlotPlan &me = hw == 0 ? s0 : s1;
        hvalid = me.valid;
        nsplit = me.nsplit;
        t0 = me.t0;
        nb_split = me.nb;
        ntail = me.ntail;
        tail_len = ntail > 0 ? (P - Pb) + p.D : 0;
        ntail_all = max(s0.ntail, s1.ntail);
        nb_all = max(s0.nb, s1.nb);
        merged = s0.valid && s1.valid && s0.unit == s1.unit;
    }
    floatx16 o[MB];
#pragma unroll
    for (int mb = 0; mb < MB; ++mb) o[mb] = floatx16{};
    float m_run = -INFINITY;
    float l_run = 0.f;

    // Tail tiles: the last P % TK cache positions followed by the D block slots,
    // zero past the end (in the unit's last split).  K and V rows, of the
    // cache or of the block ([slot][Hkv][d]), are gathered as 16-byte units
    // through registers.  All of a tail tile's loads are issued first; for the
    // first tail tile the first bulk copies follow them, so those are in
    // flight while the tail is stored and computed.
    // The first NS-1 bulk tiles into stages 0 .. NS-2 (the tail uses stage NS-1).
    auto first_fill = [&]() __attribute__((always_inline)) {
        if (nb_split > 0) {
#pragma unroll
            for (int i = 0; i < NS - 1; ++i) issue_bulk(t0 + i, i, i < nb_split);
        }
    };
    auto load_tail = [&](int st, int tt, bool fill) __attribute__((always_inline)) {
        u32x4 kr[LK], vr[LV];
#pragma unroll
        for (int i = 0; i < LK; ++i) {
            const int u = tid + i * NT;
            const int key = u / KU, lu = u % KU;
            const int j = tt * TK + key;
            const int pos = Pb + j;
            u32x4 kv = u32x4{0u, 0u, 0u, 0u}, vv = kv;
            if (j < tail_len) {
                const size_t off = pos < P ? kc_base + (size_t)pos * HD * EB + lu * 16
                                           : (((size_t)it * p.D + (pos - P)) * p.Hkv + g) * HD * EB + lu * 16;
                kv = *reinterpret_cast<const u32x4 *>((pos < P ? p.kc : p.kb) + off);
                vv = *reinterpret_cast<const u32x4 *>((pos < P ? p.vc : p.vb) + off);
            }
            kr[i] = kv;
            vr[i] = vv;
        }
        if (fill) first_fill();  // in flight while the tail is stored and computed
#pragma unroll
        for (int i = 0; i < LK; ++i) {
            const int u = tid + i * NT;
            const int key = u / KU, lu = u % KU;
            *reinterpret_cast<u32x4 *>(kbuf(st) + k_at(key, lu)) = kr[i];
            *reinterpret_cast<u32x4 *>(vbuf(st) + v_at(key, lu)) = vr[i];
        }
    };

    // S^T = K . Q^T for the tile in stage st.
    auto qk = [&](int st, floatx16 (&s)[KB]) __attribute__((always_inline)) {
        const uint8_t *Kt = kbuf(st);
#pragma unroll
        for (int kb = 0; kb < KB; ++kb) {
            s[kb] = floatx16{};
            const int key = kb * 32 + (KV8 ? key_perm8(col) : key_perm(col));
            if constexpr (!KV8) {
#pragma unroll
                for (int kc = 0; kc < KC; ++kc) {
                    const bf16x8 a = *reinterpret_cast<const bf16x8 *>(Kt + k_at(key, kc * 2 + half));
                    s[kb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, qf[kc], s[kb], 0, 0, 0);
                }
            } else {
#pragma unroll
                for (int m = 0; m < KC / 2; ++m) {
                    const u32x4 raw = *reinterpret_cast<const u32x4 *>(Kt + k_at(key, m * 2 + half));
                    s[kb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(bd_e4m3x8_to_bf16(raw.x, raw.y), qf[2 * m], s[kb], 0, 0, 0);
                    s[kb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(bd_e4m3x8_to_bf16(raw.z, raw.w), qf[2 * m + 1], s[kb], 0, 0, 0);
                }
            }
        }
    };
    // Scores a row may not use become -inf: tail tiles (tt >= 0) of the block
    // modes, or a masked tile of the sequence mode (first key mkey0 >= 0).
    auto apply_mask = [&](floatx16 (&s)[KB], int tt, int mkey0) __attribute__((always_inline)) {
        if (SEQ && mkey0 >= 0) {
#pragma unroll
            for (int kb = 0; kb < KB; ++kb)
#pragma unroll
                for (int i = 0; i < 16; ++i) {
                    const int kin = 16 * (i >> 3) + 8 * half + (i & 7);
                    s[kb][i] = in_ranges(vis, mkey0 + kb * 32 + kin) ? s[kb][i] : -INFINITY;
                }
        }
        if (!SEQ && tt >= 0) {
#pragma unroll
            for (int kb = 0; kb < KB; ++kb)
#pragma unroll
                for (int i = 0; i < 16; ++i) {
                    const int kin = KV8 ? 16 * half + i : 16 * (i >> 3) + 8 * half + (i & 7);
                    const int j = tt * TK + kb * 32 + kin;
                    const int b = Pb + j - P;  // block slot (a cache position if < 0)
                    const bool ok = (j < tail_len) & in_ranges(vis, b);
                    s[kb][i] = ok ? s[kb][i] : -INFINITY;
                }
        }
    };
    // Online softmax of one tile's scores and O^T += V^T . P^T.
    auto softmax_pv = [&](int st, floatx16 (&s)[KB]) __attribute__((always_inline)) {
        const uint8_t *Vt = vbuf(st);
        // A operands of O^T += V^T . P^T: lane (col, half) needs d = 32 mb + col
        // of the 8 keys that pb pairs with it, read by transpose loads at the
        // lane offsets v_lane[mb] plus a row offset known at compile time.  All
        // of the tile's reads are issued here, ahead of the softmax, which
        // covers their latency.
        constexpr int VR = KV8 ? C4 : 2 * C4;  // 8-byte reads per d-block
        uint32_t vraw[MB][VR][2];
#pragma unroll
        for (int mb = 0; mb < MB; ++mb)
#pragma unroll
            for (int i = 0; i < VR; ++i) {
                // bf16: read i covers keys 4 i .. 4 i + 3 of the lane's 16-key chunk
                // i / 2 rows; E4M3: keys 8 i .. (rows 32 (i / 2) + 8 (i % 2)).
                const int row = KV8 ? 32 * (i >> 1) + 8 * (i & 1) : 16 * (i >> 1) + 4 * (i & 1);
                if constexpr (!KV8) {
                    const bd_s16x4 r = bd_lds_tr16(Vt + v_lane[mb] + row * KU * 16);
                    const bd_i32x2 w = __builtin_bit_cast(bd_i32x2, r);
                    vraw[mb][i][0] = (uint32_t)w[0];
                    vraw[mb][i][1] = (uint32_t)w[1];
                } else {
                    const bd_i32x2 w = bd_lds_tr8(Vt + v_lane[mb] + row * KU * 16);
                    vraw[mb][i][0] = (uint32_t)w[0];
                    vraw[mb][i][1] = (uint32_t)w[1];
                }
            }
        float mx = -INFINITY;
#pragma unroll
        for (int kb = 0; kb < KB; ++kb)
#pragma unroll
            for (int i = 0; i < 16; ++i) mx = fmaxf(mx, s[kb][i]);
        mx = bd_max_halves(mx);
        const float mx2 = mx * cs;
        const bool need = mx2 > m_run + 8.0f;
        if (bd_wave_any(need)) {
            const float m_new = need ? mx2 : m_run;
            const float alpha = need ? bd_exp2(m_run - m_new) : 1.0f;
            l_run *= alpha;
#pragma unroll
            for (int mb = 0; mb < MB; ++mb) o[mb] *= alpha;
            m_run = m_new;
        }
        const float msub = (m_run == -INFINITY) ? 0.f : m_run;
        bf16x8 pb[C4];
#pragma unroll
        for (int kb = 0; kb < KB; ++kb)
#pragma unroll
            for (int i = 0; i < 16; ++i) pb[kb * 2 + (i >> 3)][i & 7] = (__bf16)bd_exp2(fmaf(s[kb][i], cs, -msub));
        // Row sum of the rounded weights (exactly what the P.V product uses),
        // two at a time with v_dot2_f32_bf16.
        const bf16x2 ones = {(__bf16)1.0f, (__bf16)1.0f};
        float lsum = 0.f;
#pragma unroll
        for (int c4 = 0; c4 < C4; ++c4)
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const bf16x2 pr = {pb[c4][2 * e], pb[c4][2 * e + 1]};
                lsum = __builtin_amdgcn_fdot2_f32_bf16(pr, ones, lsum, false);
            }
        l_run += lsum;
#pragma unroll
        for (int mb = 0; mb < MB; ++mb) {
#pragma unroll
            for (int c4 = 0; c4 < C4; ++c4) {
                bf16x8 a;
                if constexpr (!KV8) {
                    const u32x4 w = {vraw[mb][2 * c4][0], vraw[mb][2 * c4][1], vraw[mb][2 * c4 + 1][0],
                                     vraw[mb][2 * c4 + 1][1]};
                    a = __builtin_bit_cast(bf16x8, w);
                } else {
                    a = bd_e4m3x8_to_bf16(vraw[mb][c4][0], vraw[mb][c4][1]);
                }
                o[mb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, pb[c4], o[mb], 0, 0, 0);
            }
        }
    };
    auto compute = [&](int st, int tt /* tail tile index, -1 for bulk */,
                       int mkey0 /* sequence mode: first key of a masked tile, else -1 */) __attribute__((always_inline)) {
        floatx16 s[KB];
        qk(st, s);
        apply_mask(s, tt, mkey0);
        softmax_pv(st, s);
    };

    // Tail split: gather and compute its (one to three) tiles in stage NS-1.
    if constexpr (PAIR) {
        // A half without a tail starts its bulk copies first and only keeps
        // step with its partner's tail barriers.
        const bool spec_hit = spec && hvalid && ntail == 0 && t0 == spec_t0 && nb_split == spec_nb;
        if (spec && !spec_hit) bd_wait_vmcnt<0>();  // copies of another plan: let them land, then refill
        if (ntail == 0 && !spec_hit) first_fill();
        for (int tt = 0; tt < ntail_all; ++tt) {
            if (tt > 0) bd_barrier_lds();
            if (tt < ntail) load_tail(NS - 1, tt, tt == 0);
            bd_barrier_lds();
            if (tt < ntail && wave_active) compute(NS - 1, tt, -1);
        }
    } else {
        for (int tt = 0; tt < ntail; ++tt) {
            if (tt > 0) bd_barrier_lds();  // every wave is done with the previous tail tile
            load_tail(NS - 1, tt, tt == 0);
            bd_barrier_lds();
            if (wave_active) compute(NS - 1, tt, -1);
        }
        if (ntail == 0) first_fill();
    }
    // Bulk tiles through NS stages, NS-1 filled up front: tiles tl+1 ..
    // tl+NS-1 are in flight while tile tl is computed.  Every step has the same
    // shape - wait for all but the last NS-2 copy groups, one barrier (after
    // which no wave still reads tile tl-1's stage), refill that stage with tile
    // tl+NS-1, compute tile tl - and the
    // step count is rounded up to a multiple of NS, with dummy copy groups
    // (each lane reading one fixed, cached 16-byte unit into a stage nobody
    // reads) past the split's last tile.  The compiler can then prove that a
    // stage's reads never wait for copies into the other stages; with a
    // varying count it falls back to draining every copy before each tile.
    // The Q loads, issued before the first copies, are retired by the first
    // fixed-count wait.
    const int nb_round = (nb_all + NS - 1) / NS * NS;
    auto step = [&](auto stage, int tl) __attribute__((always_inline)) {
        constexpr int ST = decltype(stage)::value;
        bd_wait_vmcnt<(NS - 2) * (LK + LV)>();  // tile tl's copies have landed
        bd_barrier_lds();  // ... and are visible to every wave, which is done with tile tl - 1
        issue_bulk(t0 + tl + NS - 1, (ST + NS - 1) % NS, tl + NS - 1 < nb_split);  // into tile tl - 1's stage
        if (wave_active && tl < nb_split) compute(ST, -1, SEQ && t0 + tl >= nU ? tile_of(t0 + tl) * TK : -1);
    };
    for (int tl = 0; tl < nb_round; tl += NS) {
        step(std::integral_constant<int, 0>{}, tl);
        step(std::integral_constant<int, 1>{}, tl + 1);
        step(std::integral_constant<int, 2>{}, tl + 2);
        step(std::integral_constant<int, 3>{}, tl + 3);
    }
    if (nb_all > 0) bd_wait_vmcnt<0>();  // no copy may still target LDS when the workgroup ends

    float l_tot = bd_sum_halves(l_run);
    // Partials this unit leaves: its split count, less the slots absorbed by a
    // paired half (slot s >= 1 whose list index is odd: its partner s - 1 is in
    // the same workgroup and unit).
    int eff = nsplit;
    if constexpr (PAIR) {
        const int base0 = unit * p.max_splits;
        eff = nsplit - ((base0 & 1) ? (nsplit - 1) / 2 : nsplit / 2);
        if (merged) {
            // Half 1 hands its (m, l, o) to half 0 through LDS: wave w's 64
            // accumulators of each lane in lds_k<w> ([register][lane], so each
            // store of a wave fills 256 contiguous bytes), (m, l) in lds_v<w>.
            // Lane and wave layouts are the same in both halves.
            static_assert(MB * 16 * 64 * 4 <= SB * NH && NW <= NS, "exchange must fit one stage array per wave");
            bd_barrier_lds();  // every copy has landed and no wave still reads a stage
            float *xo = reinterpret_cast<float *>(kraw(w));
            float *xm = reinterpret_cast<float *>(vraw(w));
            if (hw == 1 && wave_active) {
#pragma unroll
                for (int mb = 0; mb < MB; ++mb)
#pragma unroll
                    for (int i = 0; i < 16; ++i) xo[(mb * 16 + i) * 64 + lane] = o[mb][i];
                xm[lane] = m_run;
                xm[64 + lane] = l_tot;
            }
            bd_barrier_lds();
            if (hw == 1) return;
            if (wave_active) {
                // Fixed order: this half's keys come first in the unit.
                const float m1 = xm[lane], l1 = xm[64 + lane];
                const float M = fmaxf(m_run, m1);
                const float a0 = m_run == -INFINITY ? 0.f : bd_exp2(m_run - M);
                const float a1 = m1 == -INFINITY ? 0.f : bd_exp2(m1 - M);
                l_tot = l_tot * a0 + l1 * a1;
#pragma unroll
                for (int mb = 0; mb < MB; ++mb)
#pragma unroll
                    for (int i = 0; i < 16; ++i) o[mb][i] = o[mb][i] * a0 + xo[(mb * 16 + i) * 64 + lane] * a1;
                m_run = M;
            }
        }
        if (!hvalid) return;
    }
    // Output element mapping of the O^T accumulators: block mb, register i of
    // half h holds d = mb*32 + 8*(i/4) + 4*h + (i%4) of this lane's row.
    if (eff == 1) {
        if (row_valid) {
            const float inv = l_tot > 0.f ? vs / l_tot : 0.f;  // a row that sees nothing outputs 0
            uint16_t *op = p.out + (((size_t)it * p.D + slot) * p.Hq + head) * HD;
#pragma unroll
            for (int mb = 0; mb < MB; ++mb)
#pragma unroll
                for (int i4 = 0; i4 < 4; ++i4) {
                    const int dd = mb * 32 + 8 * i4 + 4 * half;
                    uint2 v;
                    v.x = bd_f32_to_bf16(o[mb][4 * i4 + 0] * inv) | ((uint32_t)bd_f32_to_bf16(o[mb][4 * i4 + 1] * inv) << 16);
                    v.y = bd_f32_to_bf16(o[mb][4 * i4 + 2] * inv) | ((uint32_t)bd_f32_to_bf16(o[mb][4 * i4 + 3] * inv) << 16);
                    bd_store_nt(op + dd, v);
                }
        }
        return;
    }

    // Split-K partials: the split's normalised output o / l (times the V scale)
    // as bf16 plus its (m, l) in fp32, stored lane-major so that every store of
    // a wave covers one contiguous span.  16-byte unit qq (output quads 2qq and
    // 2qq+1, i.e. block mb = qq/2, quads i4 = 2(qq%2) and 2(qq%2)+1) of thread t
    // of split s of unit u lives at [(u * max_splits + s) * (QUADS/2) + qq][t].
    // They are stored write-through (sc1): the merge kernel, next on the
    // stream, then reads them from the last-level cache (non-temporal stores
    // measured slower there), and the L2 holds nothing dirty for the
    // kernel-end write-back.
    constexpr int QUADS = MB * 4;
    if (wave_active) {
        const size_t base = ((size_t)unit * p.max_splits + split);
        const float inv = l_tot > 0.f ? vs / l_tot : 0.f;
        const __amdgpu_buffer_rsrc_t ro =
            bd_region(reinterpret_cast<uint4 *>(p.ws_o) + base * (QUADS / 2) * NT, (QUADS / 2) * NT * 16);
#pragma unroll
        for (int qq = 0; qq < QUADS / 2; ++qq) {
            const int mb = qq >> 1, i0 = 8 * (qq & 1);
            uint4 v;
            v.x = bd_f32_to_bf16(o[mb][i0 + 0] * inv) | ((uint32_t)bd_f32_to_bf16(o[mb][i0 + 1] * inv) << 16);
            v.y = bd_f32_to_bf16(o[mb][i0 + 2] * inv) | ((uint32_t)bd_f32_to_bf16(o[mb][i0 + 3] * inv) << 16);
            v.z = bd_f32_to_bf16(o[mb][i0 + 4] * inv) | ((uint32_t)bd_f32_to_bf16(o[mb][i0 + 5] * inv) << 16);
            v.w = bd_f32_to_bf16(o[mb][i0 + 6] * inv) | ((uint32_t)bd_f32_to_bf16(o[mb][i0 + 7] * inv) << 16);
            bd_store_wt(ro, (unsigned)(qq * NT + tid) * 16u, v);
        }
        bd_store_wt(bd_region(p.ws_ml + base * NT, NT * 8), (unsigned)tid * 8u, make_float2(m_run, l_tot));
    }
}

// Waves per merge block: each merges one (unit, 32-row group, column part)
// per wave, so a launch has NP / kMergeWaves blocks per row group.
constexpr int kMergeWaves = 1;
// The merge grid, units * nw * (NP / kMergeWaves) with nw >= 4 and NP >= 4,
// must be a multiple of 8 for the XCD-aware block decode.
static_assert((4 * (4 / kMergeWaves)) % 8 == 0, "merge grid must be a multiple of 8");

// Merge of the split-K partials (second launch; the kernel boundary orders
// the partial stores before these loads).  Each wave of a block handles one
// (unit, 32-row group, part jq of NP column parts): the group's rows are the
// rows one wave of the tile kernel owned.  Wave j, lane `lane` merges 16-byte
// partial units qq = jq * QPT .. of lane `lane` of that wave:
//   M = max_s m_s,  c_s = 2^(m_s - M) l_s,  o = sum_s c_s (o_s / l_s) / sum_s c_s,
// summed in split order.  The merged rows are staged in LDS and written out
// as row segments of WPB * HD / NP contiguous elements.  Every split slot of a
// lane is loaded at once, QPT * MAXS 16-byte units: NP = 4 with up to 16
// splits, or one unit per split (NP = HD / 16) with up to 32.  With SW > 1
// split waves a block holds up to SW * MAXS splits: wave w takes splits
// MAXS w .. MAXS w + MAXS - 1, all use the max over all splits, and wave 0
// adds the other waves' sums to its own in wave order (the sum over its own
// splits, then each later group's).
// PAIRED: the partials of paired tile halves (some slots absorbed, see below).
template <int HD, int NW, int TK, bool SEQ, int NP, int MAXS, int SW, bool PAIRED = false>
__global__ __launch_bounds__(kMergeWaves * SW * 64) void attn_merge_kernel(MfmaParams p) {
    constexpr int WPB = kMergeWaves;    // waves per block
    constexpr int NT_TILE = NW * 64;    // threads of the tile kernel's block
    constexpr int MB = HD / 32;
    constexpr int QQ = MB * 2;          // 16-byte partial units per lane
    constexpr int QPT = QQ / NP;        // units per thread here
    constexpr int DQ = HD / NP;         // output columns of one part (QPT units)
    static_assert(QPT >= 1 && QQ % NP == 0 && MAXS * SW <= kMaxSplits, "merge shape");
    static_assert(SW == 1 || WPB == 1, "split waves take one column part per block");
    constexpr int RS = DQ * WPB + 8;    // LDS row stride (elements), staggers banks
    __shared__ __attribute__((aligned(16))) uint16_t rows_lds[32 * RS];
    // Block = (unit, wave wv of the tile kernel's block, WPB of its NP column parts).
    constexpr int QB = NP / WPB;        // blocks per (unit, wave)
    // XCD-aware decode (the grid is a multiple of 16): a unit's blocks share an
    // XCD, so the column parts of a row group fetch its (m, l) pairs
    // through one L2.
    const int lb = (blockIdx.x & 7) * (gridDim.x >> 3) + (blockIdx.x >> 3);
    const int unit = lb / (NW * QB);
    const int rem = lb - unit * (NW * QB);
    const int wv = rem / QB;
    const int qb = rem - wv * QB;
    const int rb = unit % p.row_blocks;
    const int pair = unit / p.row_blocks;
    const int g = pair % p.Hkv;
    const int it = pair / p.Hkv;
    const int row0 = rb * (NW * 32) + wv * 32;
    if (row0 >= p.R) return;
    const int tid = threadIdx.x;
    const int lane = tid & 63, half = lane >> 5, col = lane & 31;
    const int jl = SW > 1 ? 0 : tid >> 6;   // column part within the block
    const int sw = SW > 1 ? tid >> 6 : 0;   // split wave: splits MAXS sw ..
    const int jq = qb * WPB + jl;           // column part of this thread
    const int src_t = wv * 64 + lane;      // thread of the tile kernel's block
    const size_t base = (size_t)unit * p.max_splits + (size_t)sw * MAXS;
    const uint4 *wo = reinterpret_cast<const uint4 *>(p.ws_o);
    // Every workspace slot of the unit is requested before the prefix length
    // (which decides how many of them hold this call's partials) arrives;
    // slots past the unit's split count are read but not used.  A balanced
    // plan (up to twice the average split count per unit) first reads the
    // count that the unit's first split stored and requests only those slots.
    int slots_to_load = p.max_splits, nsplit_b = 0;
    if (!SEQ && p.balanced) {
        nsplit_b = p.unit_splits[unit];
        slots_to_load = nsplit_b;
    }
    // Paired halves: slot s >= 1 with an odd list index was absorbed by slot
    // s - 1 (same workgroup, same unit) and holds nothing of this call.
    const int list0 = unit * p.max_splits;
    auto absorbed = [&](int s) __attribute__((always_inline)) { return PAIRED && s >= 1 && ((list0 + s) & 1); };
    float2 ml[MAXS];
    uint4 v[QPT][MAXS];
#pragma unroll
    for (int s = 0; s < MAXS; ++s) {
        if (PAIRED) ml[s] = make_float2(-INFINITY, 0.f);
        if (sw * MAXS + s < slots_to_load && !absorbed(sw * MAXS + s)) {
            // Each partial is read once: non-temporal loads.
            const floatx2_nt m2 =
                __builtin_nontemporal_load(reinterpret_cast<const floatx2_nt *>(p.ws_ml) + (base + s) * NT_TILE + src_t);
            ml[s] = make_float2(m2[0], m2[1]);
#pragma unroll
            for (int j = 0; j < QPT; ++j) {
                const u32x4 t = __builtin_nontemporal_load(reinterpret_cast<const u32x4 *>(wo) +
                                                           ((base + s) * QQ + jq * QPT + j) * NT_TILE + src_t);
                v[j][s] = make_uint4(t[0], t[1], t[2], t[3]);
            }
        }
    }
    int nsplit;
    if constexpr (SEQ) {
        nsplit = p.unit_splits[unit];  // written by the unit's first split
    } else if (p.balanced) {
        nsplit = nsplit_b;
    } else {
        const int P = min(max(p.prefix[it], 0), p.cap);
        nsplit = unit_nsplit<TK>(P, p.D, p.tiles_per_split, p.max_splits);
    }
    // A unit left with one partial was written out by the tile kernel.
    const int eff = PAIRED ? nsplit - ((list0 & 1) ? (nsplit - 1) / 2 : nsplit / 2) : nsplit;
    if (eff == 1) return;
    const int ns = nsplit - sw * MAXS;  // splits of this wave (may be <= 0)
    float M = -INFINITY;
#pragma unroll
    for (int s = 0; s < MAXS; ++s)
        if (s < ns && !absorbed(sw * MAXS + s)) M = fmaxf(M, ml[s].x);
    if constexpr (SW > 1) {
        __shared__ float m_x[SW][64];
        m_x[sw][lane] = M;
        __syncthreads();
#pragma unroll
        for (int w = 0; w < SW; ++w) M = fmaxf(M, m_x[w][lane]);
    }
    float L = 0.f;
    float acc[QPT][8] = {};
#pragma unroll
    for (int s = 0; s < MAXS; ++s)
        if (s < ns && !absorbed(sw * MAXS + s)) {
            const float c = (ml[s].x == -INFINITY) ? 0.f : bd_exp2(ml[s].x - M) * ml[s].y;
            L += c;
#pragma unroll
            for (int j = 0; j < QPT; ++j) {
                const uint32_t w4[4] = {v[j][s].x, v[j][s].y, v[j][s].z, v[j][s].w};
#pragma unroll
                for (int e = 0; e < 8; ++e)
                    acc[j][e] += c * bd_bf16_to_f32((uint16_t)(w4[e >> 1] >> (16 * (e & 1))));
            }
        }
    if constexpr (SW > 1) {
        __shared__ float sum_x[SW][QPT * 8 + 1][64];
        sum_x[sw][0][lane] = L;
#pragma unroll
        for (int j = 0; j < QPT; ++j)
#pragma unroll
            for (int e = 0; e < 8; ++e) sum_x[sw][1 + j * 8 + e][lane] = acc[j][e];
        __syncthreads();
        if (sw == 0) {
#pragma unroll
            for (int w = 1; w < SW; ++w) {
                L += sum_x[w][0][lane];
#pragma unroll
                for (int j = 0; j < QPT; ++j)
#pragma unroll
                    for (int e = 0; e < 8; ++e) acc[j][e] += sum_x[w][1 + j * 8 + e][lane];
            }
        }
    }
    const float inv = L > 0.f ? 1.0f / L : 0.f;
    // Unit qq holds d = mb*32 + 16*(qq%2) + 4*half + {0..3} and the same + 8;
    // in this block's LDS rows, column d - qb * WPB * DQ.  With split waves,
    // wave 0 alone holds the sums and writes the rows.
#pragma unroll
    for (int j = 0; j < QPT; ++j) {
        if (sw != 0) continue;
        const int qq = jq * QPT + j;
        const int d0 = (qq >> 1) * 32 + 16 * (qq & 1) + 4 * half - qb * WPB * DQ;
#pragma unroll
        for (int h8 = 0; h8 < 2; ++h8) {
            uint2 o;
            o.x = bd_f32_to_bf16(acc[j][4 * h8 + 0] * inv) | ((uint32_t)bd_f32_to_bf16(acc[j][4 * h8 + 1] * inv) << 16);
            o.y = bd_f32_to_bf16(acc[j][4 * h8 + 2] * inv) | ((uint32_t)bd_f32_to_bf16(acc[j][4 * h8 + 3] * inv) << 16);
            *reinterpret_cast<uint2 *>(&rows_lds[col * RS + d0 + 8 * h8]) = o;
        }
    }
    __syncthreads();
    if (sw != 0) return;
    // The block's columns of each row out: TPR threads per row, 16 bytes each.
    constexpr int TPR = WPB * DQ / 8;
    constexpr int RPP = WPB * 64 / TPR;  // rows per pass
#pragma unroll
    for (int r0 = 0; r0 < 32; r0 += RPP) {
        const int rr = r0 + tid / TPR, u = tid % TPR;
        const int r = row0 + rr;
        if (r < p.R) {
            const int slot = r / p.G;
            const int head = g * p.G + (r - slot * p.G);
            uint16_t *op = p.out + (((size_t)it * p.D + slot) * p.Hq + head) * HD + qb * WPB * DQ + u * 8;
            bd_store_nt(op, *reinterpret_cast<const uint4 *>(&rows_lds[rr * RS + u * 8]));
        }
    }
}

// ---------------------------------------------------------------------------
// Vector path: one wave per (item, slot, head) query row, keys 64 at a time
// across lanes, values accumulated with lanes over d.  Used for fp32 inputs.
// ---------------------------------------------------------------------------
template <typename T>
__device__ __forceinline__ float ld(const T *p, size_t i);
template <>
__device__ __forceinline__ float ld<float>(const float *p, size_t i) { return p[i]; }
template <>
__device__ __forceinline__ float ld<uint16_t>(const uint16_t *p, size_t i) { return bd_bf16_to_f32(p[i]); }
__device__ __forceinline__ void st(float *p, size_t i, float v) { p[i] = v; }
__device__ __forceinline__ void st(uint16_t *p, size_t i, float v) { p[i] = bd_f32_to_bf16(v); }

template <typename T, int HD>
__global__ __launch_bounds__(256) void attn_vec_kernel(const T *q, const T *kb, const T *vb, const T *kc,
                                                       const T *vc, const int32_t *prefix, T *out, int n,
                                                       int D, int Hq, int Hkv, int cap, int mode, int B, float scale) {
    constexpr int PER = HD / 64;
    __shared__ float qs[4][HD];
    const int lane = threadIdx.x & 63;
    const int w = threadIdx.x >> 6;
    const long u = (long)blockIdx.x * 4 + w;
    const bool active = u < (long)n * D * Hq;
    const int it = active ? (int)(u / ((long)D * Hq)) : 0;
    const int slot = (int)((u / Hq) % D);
    const int h = (int)(u % Hq);
    const int g = h / (Hq / Hkv);
    const size_t qoff = (((size_t)it * D + slot) * Hq + h) * HD;
    for (int t = lane; t < HD; t += 64) qs[w][t] = active ? ld(q, qoff + t) : 0.f;
    __syncthreads();
    if (!active) return;
    const int P = min(max(prefix[it], 0), cap);
    const int nk = P + D;
    const SlotRanges vis = block_ranges(mode, slot, D, B);
    const size_t kc_base = ((size_t)it * Hkv + g) * cap * HD;  // K and V cache rows [cap][HD]
    float m = -INFINITY, l = 0.f, o[PER];
#pragma unroll
    for (int e = 0; e < PER; ++e) o[e] = 0.f;
    for (int base = 0; base < nk; base += 64) {
        const int key = base + lane;
        const bool valid = (key < nk) & in_ranges(vis, key - P);
        float s = -INFINITY;
        if (valid) {
            float acc = 0.f;
            if (key < P) {
                for (int t = 0; t < HD; ++t) acc = fmaf(qs[w][t], ld(kc, kc_base + (size_t)key * HD + t), acc);
            } else {
                const size_t kbo = (((size_t)it * D + (key - P)) * Hkv + g) * HD;
                for (int t = 0; t < HD; ++t) acc = fmaf(qs[w][t], ld(kb, kbo + t), acc);
            }
            s = acc * scale;
        }
        float mx = s;
        for (int off = 32; off >= 1; off >>= 1) mx = fmaxf(mx, __shfl_xor(mx, off, 64));
        const float m_new = fmaxf(m, mx);
        const float alpha = (m == -INFINITY) ? 0.f : expf(m - m_new);
        const float pv = valid ? expf(s - m_new) : 0.f;
        float ps = pv;
        for (int off = 32; off >= 1; off >>= 1) ps += __shfl_xor(ps, off, 64);
        l = l * alpha + ps;
#pragma unroll
        for (int e = 0; e < PER; ++e) o[e] *= alpha;
        m = m_new;
        const int kmax = min(64, nk - base);
        for (int kk = 0; kk < kmax; ++kk) {
            const float pk = __shfl(pv, kk, 64);
            if (pk == 0.f) continue;
            const int key2 = base + kk;
#pragma unroll
            for (int e = 0; e < PER; ++e) {
                const int dd = lane + 64 * e;
                const float vv = key2 < P ? ld(vc, kc_base + (size_t)key2 * HD + dd)
                                          : ld(vb, (((size_t)it * D + (key2 - P)) * Hkv + g) * HD + dd);
                o[e] = fmaf(pk, vv, o[e]);
            }
        }
    }
#pragma unroll
    for (int e = 0; e < PER; ++e) st(out, qoff + lane + 64 * e, o[e] / l);
}

}  // namespace

AttnPlan plan_attention(int n, int D, int Hq, int Hkv, int d, int dtype, int max_prefix, bool seq, bool balanced) {
    AttnPlan pl{};
    pl.seq = seq;
    pl.max_prefix = max_prefix;
    pl.mfma = (dtype == 1 || dtype == 2);
    pl.fp8 = (dtype == 2);
    pl.tk = pl.fp8 ? 2 * kTileKeys : kTileKeys;
    pl.rows = D * (Hq / Hkv);
    if (!pl.mfma) {
        pl.grid = (int)(((long)n * D * Hq + 3) / 4);
        pl.ws_bytes = 0;
        return pl;
    }
    // 8-wave workgroups (256 rows) only for d = 128: with d = 64 a tile has
    // fewer 16-byte units than 8 waves have lanes.  The two-stream mode keeps
    // 4-wave workgroups (two per CU, so the two waves of a SIMD belong to
    // different workgroups and their MFMA and softmax phases drift apart;
    // its many units fill the GPU either way): 396-399 against 405-406 us.
    pl.nw = (pl.rows <= 128 || d == 64 || seq) ? 4 : 8;
    pl.rows_per_group = pl.nw * 32;
    pl.row_blocks = (pl.rows + pl.rows_per_group - 1) / pl.rows_per_group;
    pl.units = n * Hkv * pl.row_blocks;
    // Workgroups to launch: as many as hold two waves per SIMD.  LDS (kStages
    // tile stages) allows two workgroups per CU, which is that many for 4-wave
    // workgroups; 8-wave workgroups are sized for one per CU, since a second one
    // (four waves per SIMD) slowed the 8-item 7B step by 15%.
    const int slots = kCUs * occupancy_for(d) * 4 / pl.nw;
    const int ntiles_max = max_prefix / pl.tk;
    const int want = std::max(1, slots / pl.units);
    // Splits per unit (the device side derives each unit's count from its own
    // prefix): sized so that a unit at max_prefix gets about `want` splits, at
    // most kNarrowSplits; up to kWideSplits or kMaxSplits while each workgroup
    // still has a CU of its own (few units, where a lone wave per SIMD makes
    // the tile loop latency-bound and shorter splits pay).
    // kMaxSplits only where each split keeps two bulk tiles or more: with one
    // the tail split and the larger merge cost more than the shorter splits save.
    const int cap = (long)pl.units * kMaxSplits <= kCUs && ntiles_max >= 2 * kMaxSplits ? kMaxSplits
                    : (long)pl.units * kWideSplits <= kCUs                               ? kWideSplits
                                                                                          : kNarrowSplits;
    pl.max_splits = ntiles_max == 0 ? 1 : std::max(2, std::min(std::min(want, ntiles_max + 1), cap));
    // Work of a unit at max_prefix in bulk-tile units: its bulk tiles plus
    // kTailCost per tail tile (up to tk - 1 cache positions and the D slots).
    const int ntail_max = (pl.tk - 1 + D + pl.tk - 1) / pl.tk;
    const int work_max = ntiles_max + kTailCost * ntail_max;
    pl.tiles_per_split = std::max(1, (work_max + pl.max_splits - 1) / pl.max_splits);
    // Ragged batch (caller's hint): the device balances split counts across
    // items from their prefix lengths, each unit getting up to twice the
    // average (at most the cap above), within the same number of workgroups.
    if (balanced && !seq && n <= kBalancedMaxItems && ntiles_max >= 1 && pl.units <= slots) {
        pl.balanced = true;
        pl.balance_slots = slots;
        pl.max_splits = std::max(2, std::min(std::min(2 * want, cap), ntiles_max + 1));
        pl.tiles_per_split = 1;  // unused: the device plan sets each unit's split count
    }
    if (seq) {
        // Whole sequences of D positions: a unit has at most D / tk key tiles,
        // all streamed the same way; the split count only fills the GPU.
        const int nt = (D + pl.tk - 1) / pl.tk;
        pl.max_splits = std::max(1, std::min(std::min(want, nt), cap));
        pl.tiles_per_split = std::max(1, (nt + pl.max_splits - 1) / pl.max_splits);
    }
    // Where two 4-wave workgroups would share every CU (d = 128 block modes
    // with the fixed split plan), one 8-wave workgroup runs two list slots.
    pl.pair = BD_PAIR_HALVES && !seq && !pl.balanced && pl.nw == 4 && d == 128 && pl.max_splits > 1 &&
              pl.max_splits <= kNarrowSplits && (long)pl.units * pl.max_splits > kCUs;
    const long total = pl.balanced ? (long)pl.balance_slots : (long)pl.units * pl.max_splits;
    pl.grid = (int)(((pl.pair ? (total + 1) / 2 : total) + 7) / 8 * 8);
    if (pl.max_splits > 1) {
        size_t off = 0;
        auto take = [&](size_t bytes) {
            size_t o = off;
            off += (bytes + 255) / 256 * 256;
            return o;
        };
        // Per (unit, split): every thread of the workgroup stores d/2 bf16
        // outputs of the split (normalised) plus one fp32 (m, l) pair.
        const size_t lanes = (size_t)pl.units * pl.max_splits * pl.nw * 64;
        pl.ws_ml_off = take(sizeof(float) * 2 * lanes);
        pl.ws_o_off = take(sizeof(uint16_t) * (size_t)(d / 2) * lanes);
        if (seq || pl.balanced) pl.ws_splits_off = take(sizeof(int) * (size_t)pl.units);
        pl.ws_bytes = off;
    }
    return pl;
}

namespace {
// Split waves of the merge for plans beyond kWideSplits splits (one-item
// calls): eight waves of kMaxSplits / 8 slots each, so a block has four times
// the loads in flight that two 32-slot waves had (a step of 36 one-layer
// calls of the 3B shape: 518 us with two waves, 493 with four, 487 with
// eight, 492 with sixteen).
constexpr int kMaxSplitWaves = 8;
// The merge instance holds every split slot of a lane in registers: four
// column parts for up to kNarrowSplits splits, one 16-byte unit per split
// (HD / 16 parts) up to kWideSplits, and kMaxSplitWaves split waves of such
// units per block beyond.
template <int HD, int NW, int TK, bool SEQ>
const void *pick_merge(const AttnPlan &pl) {
    // Paired plans have more slots than CUs, so at most kNarrowSplits per unit.
    if constexpr (!SEQ && HD == 128 && NW == 4)
        if (pl.pair) return (const void *)attn_merge_kernel<HD, NW, TK, SEQ, 4, kNarrowSplits, 1, true>;
    if (pl.max_splits <= kNarrowSplits) return (const void *)attn_merge_kernel<HD, NW, TK, SEQ, 4, kNarrowSplits, 1>;
    if (pl.max_splits <= kWideSplits) return (const void *)attn_merge_kernel<HD, NW, TK, SEQ, HD / 16, kWideSplits, 1>;
    return (const void *)attn_merge_kernel<HD, NW, TK, SEQ, HD / 16, kMaxSplits / kMaxSplitWaves, kMaxSplitWaves>;
}
template <bool KV8, bool SEQ>
void pick_kernels(const AttnPlan &pl, int d, const void **tile, const void **merge, int *parts, int *waves) {
    constexpr int TK = KV8 ? 2 * kTileKeys : kTileKeys;
    if (d == 128) {
        if constexpr (!SEQ) {
            if (pl.pair) *tile = (const void *)attn_mfma_kernel<128, 4, KV8, false, true>;
        }
        if (!pl.pair)
            *tile = pl.nw == 4 ? (const void *)attn_mfma_kernel<128, 4, KV8, SEQ>
                               : (const void *)attn_mfma_kernel<128, 8, KV8, SEQ>;
        *merge = pl.nw == 4 ? pick_merge<128, 4, TK, SEQ>(pl) : pick_merge<128, 8, TK, SEQ>(pl);
    } else {
        *tile = (const void *)attn_mfma_kernel<64, 4, KV8, SEQ>;
        *merge = pick_merge<64, 4, TK, SEQ>(pl);
    }
    *parts = pl.max_splits <= kNarrowSplits ? 4 : d / 16;
    *waves = pl.max_splits <= kWideSplits ? 1 : kMaxSplitWaves;
}
}  // namespace

hipError_t launch_attention_mfma(const AttnPlan &pl, const AttnArgs &a, hipStream_t s) {
    MfmaParams p{};
    p.q = (const uint16_t *)a.q;
    p.kb = (const uint8_t *)a.k_blk;
    p.vb = (const uint8_t *)a.v_blk;
    p.kc = (const uint8_t *)a.k_cache;
    p.vc = (const uint8_t *)a.v_cache;
    p.prefix = a.prefix;
    p.k_scale = a.k_scale;
    p.v_scale = a.v_scale;
    p.out = (uint16_t *)a.out;
    char *ws = (char *)a.ws;
    p.ws_ml = pl.max_splits > 1 ? (float2 *)(ws + pl.ws_ml_off) : nullptr;
    p.ws_o = pl.max_splits > 1 ? (float *)(ws + pl.ws_o_off) : nullptr;
    p.unit_splits = pl.max_splits > 1 && (pl.seq || pl.balanced) ? (int *)(ws + pl.ws_splits_off) : nullptr;
    p.spans = a.spans;
    p.n_spans = a.n_spans;
    p.Lc = a.Lc;
    p.max_spans = a.max_spans;
    p.Dblk = a.Dblk;
    p.n = a.n;
    p.D = a.D;
    p.Hq = a.Hq;
    p.Hkv = a.Hkv;
    p.G = a.Hq / a.Hkv;
    p.cap = a.cap;
    p.mode = a.mode;
    p.B = a.B;
    p.R = pl.rows;
    p.row_blocks = pl.row_blocks;
    p.max_splits = pl.max_splits;
    p.tiles_per_split = pl.tiles_per_split;
    p.total_logical = pl.units * pl.max_splits;
    p.balanced = pl.balanced ? 1 : 0;
    p.balance_slots = pl.balance_slots;
    p.max_prefix = pl.max_prefix;
    p.c = a.scale * BD_LOG2E;
    dim3 block(pl.nw * 64 * (pl.pair ? 2 : 1));
    const void *tile, *merge;
    int parts, waves;
    if (pl.seq)
        pick_kernels<false, true>(pl, a.d, &tile, &merge, &parts, &waves);
    else if (pl.fp8)
        pick_kernels<true, false>(pl, a.d, &tile, &merge, &parts, &waves);
    else
        pick_kernels<false, false>(pl, a.d, &tile, &merge, &parts, &waves);
    void *args[] = {&p};
    hipError_t e = hipLaunchKernel(tile, dim3(pl.grid), block, args, 0, s);
    if (e != hipSuccess || pl.max_splits == 1) return e;
    return hipLaunchKernel(merge, dim3(pl.units * pl.nw * (parts / kMergeWaves)), dim3(kMergeWaves * waves * 64), args, 0,
                           s);
}

hipError_t launch_attention_vec(const AttnArgs &a, int dtype, hipStream_t s) {
    const long rows = (long)a.n * a.D * a.Hq;
    dim3 grid((unsigned)((rows + 3) / 4)), block(256);
    if (dtype == 0) {
        auto *q = (const float *)a.q;
        if (a.d == 128)
            hipLaunchKernelGGL((attn_vec_kernel<float, 128>), grid, block, 0, s, q, (const float *)a.k_blk,
                               (const float *)a.v_blk, (const float *)a.k_cache, (const float *)a.v_cache,
                               a.prefix, (float *)a.out, a.n, a.D, a.Hq, a.Hkv, a.cap, a.mode, a.B, a.scale);
        else
            hipLaunchKernelGGL((attn_vec_kernel<float, 64>), grid, block, 0, s, q, (const float *)a.k_blk,
                               (const float *)a.v_blk, (const float *)a.k_cache, (const float *)a.v_cache,
                               a.prefix, (float *)a.out, a.n, a.D, a.Hq, a.Hkv, a.cap, a.mode, a.B, a.scale);
    } else {
        auto *q = (const uint16_t *)a.q;
        if (a.d == 128)
            hipLaunchKernelGGL((attn_vec_kernel<uint16_t, 128>), grid, block, 0, s, q, (const uint16_t *)a.k_blk,
                               (const uint16_t *)a.v_blk, (const uint16_t *)a.k_cache,
                               (const uint16_t *)a.v_cache, a.prefix, (uint16_t *)a.out, a.n, a.D, a.Hq,
                               a.Hkv, a.cap, a.mode, a.B, a.scale);
        else
            hipLaunchKernelGGL((attn_vec_kernel<uint16_t, 64>), grid, block, 0, s, q, (const uint16_t *)a.k_blk,
                               (const uint16_t *)a.v_blk, (const uint16_t *)a.k_cache,
                               (const uint16_t *)a.v_cache, a.prefix, (uint16_t *)a.out, a.n, a.D, a.Hq,
                               a.Hkv, a.cap, a.mode, a.B, a.scale);
    }
    return hipGetLastError();
}

}  // namespace bd
