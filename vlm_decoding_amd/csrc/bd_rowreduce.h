// Row reductions shared by the vocabulary-wide kernels (confidence + commit,
// speculative verify, LM head): a running (max, first argmax, sum of
// exp(x - max)) state, its fixed-order combination across lanes, and the
// one-wave commit of a request.
//
// Confidence (DiffusionVL notes, cached block decoding): the greedy token
// a = argmax_v x_v (lowest index on ties) and its probability
// conf = 1 / sum_v exp(x_v - x_a).  Commit (Algorithm 1 and the dynamic rule
// as restated there): the k = min(ceil(D/S), |M|) most confident masked
// slots, plus every masked slot with conf > tau.
#pragma once

#include "bd_common.h"

namespace bd {

struct Part {
    float m;  // running maximum
    float s;  // sum of exp(x - m)
    int i;    // index of the first maximum
};

__device__ __forceinline__ Part combine(Part a, Part b) {
    Part r;
    const bool take_b = b.m > a.m || (b.m == a.m && b.i < a.i);
    r.m = take_b ? b.m : a.m;
    r.i = take_b ? b.i : a.i;
    const float sa = a.m == -INFINITY ? 0.f : a.s * bd_exp2((a.m - r.m) * BD_LOG2E);
    const float sb = b.m == -INFINITY ? 0.f : b.s * bd_exp2((b.m - r.m) * BD_LOG2E);
    r.s = sa + sb;
    return r;
}

template <bool WITH_SUM>
__device__ __forceinline__ void push(Part &p, float x, int idx) {
    if (x > p.m) {
        if (WITH_SUM) p.s = p.s * bd_exp2((p.m - x) * BD_LOG2E) + 1.0f;
        p.m = x;
        p.i = idx;
    } else if (WITH_SUM) {
        p.s += bd_exp2((x - p.m) * BD_LOG2E);
    }
}

// Lane exchanges without an LDS round trip.  combine() is commutative, so both
// lanes of every exchanged pair compute the same value and, after a full tree,
// every lane of the group holds the group's result.  The tree is fixed, so
// the result does not depend on timing.
template <int CTRL>  // gfx9 DPP control inside 16-lane rows
__device__ __forceinline__ Part dpp_part(Part p) {
    Part o;
    o.m = __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(p.m), CTRL, 0xf, 0xf, false));
    o.s = __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(p.s), CTRL, 0xf, 0xf, false));
    o.i = __builtin_amdgcn_update_dpp(0, p.i, CTRL, 0xf, 0xf, false);
    return combine(p, o);
}
// Reduce over the 16 lanes of each DPP row: lane ^ 1, lane ^ 2 (quad
// permutes), then the 8-lane and 16-lane mirrors.
__device__ __forceinline__ Part reduce16(Part p) {
    p = dpp_part<0xB1>(p);   // quad_perm [1,0,3,2]
    p = dpp_part<0x4E>(p);   // quad_perm [2,3,0,1]
    p = dpp_part<0x141>(p);  // row_half_mirror
    return dpp_part<0x140>(p);  // row_mirror
}
// Exchange with the lane 16 (row pair) or 32 (half) lanes away: the swap hands
// both lanes the same ordered pair (lower group's value, upper group's value).
template <bool HALVES>
__device__ __forceinline__ Part swap_part(Part p) {
    const unsigned m = __float_as_uint(p.m), s = __float_as_uint(p.s), i = (unsigned)p.i;
    const auto rm = HALVES ? __builtin_amdgcn_permlane32_swap(m, m, false, false)
                           : __builtin_amdgcn_permlane16_swap(m, m, false, false);
    const auto rs = HALVES ? __builtin_amdgcn_permlane32_swap(s, s, false, false)
                           : __builtin_amdgcn_permlane16_swap(s, s, false, false);
    const auto ri = HALVES ? __builtin_amdgcn_permlane32_swap(i, i, false, false)
                           : __builtin_amdgcn_permlane16_swap(i, i, false, false);
    return combine(Part{__uint_as_float(rm[0]), __uint_as_float(rs[0]), (int)ri[0]},
                   Part{__uint_as_float(rm[1]), __uint_as_float(rs[1]), (int)ri[1]});
}
__device__ __forceinline__ Part wave_reduce(Part p) {
    return swap_part<true>(swap_part<false>(reduce16(p)));
}

// Commit of one request by one wave (lane i = slot i, D <= 64): conf[i] and
// arg[i] (LDS) hold the merged confidence and greedy token of every masked
// slot; mask has bit i set for masked slots, nm = its popcount.  rank = the
// number of masked slots ahead in (confidence desc, index asc), read as 16-byte
// LDS broadcasts sixteen slots per round.  Writes tokens / masked for the
// committed slots and the optional outputs; returns the ballot of commits.
__device__ __forceinline__ unsigned long long commit_request(const float *conf, const int *arg, unsigned long long mask,
                                                             int nm, int D, int S, float tau, int lane, uint8_t *masked,
                                                             int32_t *tokens, float *conf_out, int32_t *argmax_out,
                                                             uint8_t *committed) {
    const bool part_i = lane < D && ((mask >> lane) & 1ull);
    const float cf = part_i ? conf[lane] : __int_as_float(0x7fc00000);
    const int am = part_i ? arg[lane] : -1;
    const int k = min((D + S - 1) / S, nm);
    int rank = 0;
    for (int j0 = 0; j0 < D; j0 += 16) {
        float cj[16];
#pragma unroll
        for (int q = 0; q < 4; ++q) {
            const float4 c4 = *reinterpret_cast<const float4 *>(&conf[j0 + 4 * q]);
            cj[4 * q] = c4.x;
            cj[4 * q + 1] = c4.y;
            cj[4 * q + 2] = c4.z;
            cj[4 * q + 3] = c4.w;
        }
        const unsigned mj = (unsigned)(mask >> j0) & 0xffffu;
        // Bitwise operators, not && / ||: no branch per slot.
#pragma unroll
        for (int e = 0; e < 16; ++e) {
            const int j = j0 + e;
            const bool ahead = (((mj >> e) & 1u) != 0) & ((cj[e] > cf) | ((cj[e] == cf) & (j < lane)));
            rank += ahead ? 1 : 0;
        }
    }
    const bool take = part_i && (rank < k || cf > tau);
    const unsigned long long tb = __builtin_amdgcn_ballot_w64(take);
    if (lane < D) {
        if (take) {
            tokens[lane] = am;
            masked[lane] = 0;
        }
        if (conf_out) conf_out[lane] = cf;
        if (argmax_out) argmax_out[lane] = am;
        if (committed) committed[lane] = take ? 1 : 0;
    }
    return tb;
}

}  // namespace bd
