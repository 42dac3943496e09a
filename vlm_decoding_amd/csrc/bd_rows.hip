// Vocab-wide row reductions on gfx950: confidence + commit, and speculative verify.
//
// Confidence (DiffusionVL notes, cached block decoding): for each masked
// slot the greedy token a = argmax_v x_v (lowest index on ties) and its
// probability conf = 1 / sum_v exp(x_v - x_a).  Commit (Algorithm 1 and the
// dynamic rule as restated there): the k = min(ceil(D/S), |M|) most
// confident masked slots, plus every masked slot with conf > tau.
// Verify (Fast-dVLM write-up, section 5.3, linear speculative decoding):
// the accepted length is the first slot whose greedy token differs from
// the draft.
//
// Work split.  Each request gets G workgroups of 256 threads (G sized by the
// host as if every slot took part).  Every workgroup first reads the
// request's masked flags (one 64-byte line) and learns the rows that take
// part - the masked slots, or every slot for verify - and their number nm.
// The G workgroups are then dealt out over those rows, cpr = G / nm chunks
// of contiguous columns per row, so every launched workgroup streams logits
// of a participating row whatever the masked set is, and no byte of an
// unmasked row is read.  A workgroup streams its chunk with 16-byte loads
// (up to 16 per thread in flight) into a running (max, index of first max,
// sum of exp(x - max)) per thread, combined in a fixed tree.
//
// Hand-off.  The finisher of a request is elected when the workgroups start:
// each takes a ticket on its group's counter (kTicketGroup workgroups; tickets
// on one address are served one after another, about 10 ns each, measured),
// the last of a group takes one on the request's counter, and the workgroup
// holding the request's last ticket finishes.  These round trips overlap the
// logits stream.  Every workgroup - idle ones included - then publishes its
// partial as two 64-bit atomic stores tagged non-zero, without waiting for
// them; the finisher polls the request's slots until all are tagged, stages
// the partials in LDS, clears the slots, merges each row's chunks in chunk
// order (16 lanes per row, a fixed tree) and runs the one-wave commit /
// verify tail.  Waiting is safe: when the finisher is known every workgroup of
// its request has taken its ticket, so has started, and none of them waits.
// A slot is published after its workgroup's masked-flag reads have returned,
// so the finisher rewrites the flags only after every reader is done.  Every
// counter has a 256-byte line of its own.  No float atomics, so results are
// identical run to run.
#include "bd_common.h"
#include "bd_internal.h"
#include "bd_rowreduce.h"

namespace bd {
namespace {

constexpr int NT = 256;
constexpr int kBatch = 16;          // 16-byte loads per thread in flight at once
#ifndef BD_ROW_WG_TARGET
#define BD_ROW_WG_TARGET 512
#endif
constexpr int kWgTarget = BD_ROW_WG_TARGET;  // workgroups a call aims for (two per CU)
constexpr int kMaxGroups = 1024;    // workgroups per request (the finisher stages their partials in LDS)
#ifndef BD_ROW_MAX_CHUNK
#define BD_ROW_MAX_CHUNK 32768
#endif
constexpr int kMaxChunk = BD_ROW_MAX_CHUNK;  // floats per workgroup, upper target when every slot takes part
constexpr int kMinChunk = 1024;     // ... lower bound of the plan (one 16-byte load per thread)
#ifndef BD_ROW_MIN_CHUNK_RUN
#define BD_ROW_MIN_CHUNK_RUN 8192
#endif
// Lower bound of a chunk when few slots take part: the plan's G workgroups
// are sized for every slot, and a row never gets more than V / kMinChunkRun
// chunks (nor fewer than the plan's own), so with few masked slots part of
// the workgroups stay idle instead of streaming slivers, and the finisher
// merges fewer partials.
constexpr int kMinChunkRun = BD_ROW_MIN_CHUNK_RUN;
constexpr int kTicketGroup = 16;    // workgroups per first-level ticket counter
constexpr int kCounterStride = 64;  // ints between counters (a 256-byte line each)
constexpr int kPollLimit = 1 << 20; // bound of the finisher's wait (rounds of loads)

struct RowParams {
    const float *logits;
    uint8_t *masked;
    int32_t *tokens;
    float *conf;
    int32_t *argmax;
    uint8_t *committed;
    int32_t *n_committed;
    const int32_t *draft;
    int32_t *accepted_len;
    uint64_t *part;   // [n_req][G][2] published partials: (max, index of the first max + 2), (sum, 1)
    int *grp_cnt;     // [n_req][NG] first-level tickets, kCounterStride apart
    int *req_cnt;     // [n_req] second-level tickets, kCounterStride apart
    int n_req, D, V, S, G, NG, max_cpr;
    float tau;
};

// Four consecutive logits (indices e..e+3) into a running state: one max over
// the four, the rare rescale only when the running maximum grows (the new
// argmax is the first of the four equal to it: every earlier element this
// thread saw is below it), then the four exponentials.
template <bool WITH_SUM>
__device__ __forceinline__ void push4(Part &acc, float4 v, int e) {
    const float lm = fmaxf(fmaxf(v.x, v.y), fmaxf(v.z, v.w));
    if (lm > acc.m) {
        const int k = v.x == lm ? 0 : v.y == lm ? 1 : v.z == lm ? 2 : 3;
        if (WITH_SUM) acc.s *= bd_exp2((acc.m - lm) * BD_LOG2E);  // 0 while acc.m is -inf
        acc.m = lm;
        acc.i = e + k;
    }
    if (WITH_SUM) {
        const float m = acc.m;
        acc.s += (bd_exp2((v.x - m) * BD_LOG2E) + bd_exp2((v.y - m) * BD_LOG2E)) +
                 (bd_exp2((v.z - m) * BD_LOG2E) + bd_exp2((v.w - m) * BD_LOG2E));
    }
}

template <bool VERIFY>
__global__ __launch_bounds__(NT) void row_kernel(RowParams p) {
    __shared__ float2 s_ms[kMaxGroups];
    __shared__ int s_i[kMaxGroups];
    __shared__ Part s_part[NT / 64];
    __shared__ __attribute__((aligned(16))) float s_conf[64];
    __shared__ int s_arg[64];
    __shared__ int s_slot[64];
    __shared__ int s_done;
    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int w = tid >> 6;
    const int r = blockIdx.x / p.G;
    const int b = blockIdx.x - r * p.G;
    const size_t ob = (size_t)r * p.D;
    const int grp = b / kTicketGroup;
    const int gsize = min(kTicketGroup, p.G - grp * kTicketGroup);
    int *gc = p.grp_cnt + ((size_t)r * p.NG + grp) * kCounterStride;
    int *rc = p.req_cnt + (size_t)r * kCounterStride;

    // Finisher election, at the start: the workgroup that takes the request's
    // last ticket (the last of its group, then the last group) finishes.  Its
    // round trips overlap the logits stream, and when it is known every other
    // workgroup of the request has started, so the finisher may wait for them.
    int tk = 0;
    if (tid == 0) tk = bd_ticket(gc);

    // The rows that take part and the j-th of them.  Each wave reads the flags
    // itself, so no barrier is needed before the loads.
    unsigned long long mask;
    if (VERIFY)
        mask = p.D == 64 ? ~0ull : (1ull << p.D) - 1ull;
    else
        mask = __builtin_amdgcn_ballot_w64(lane < p.D && p.masked[ob + lane] != 0);
    const int nm = __popcll(mask);
    // rank of this lane's slot among the participating slots
    const int rank = (int)__builtin_amdgcn_mbcnt_hi((uint32_t)(mask >> 32),
                                                    __builtin_amdgcn_mbcnt_lo((uint32_t)mask, 0u));
    const bool in_mask = (mask >> lane) & 1ull;
    const int cpr = nm == 0 ? 0 : min(p.G / nm, p.max_cpr);  // chunks per participating row
    const bool active = b < nm * cpr;
    int rq = 0;
    if (tid == 0 && tk == gsize - 1) {
        bd_coherent_store(gc, 0);  // every ticket of the group is taken: reset for the next call
        if (p.NG > 1) rq = bd_ticket(rc);
    }

    Part acc{-INFINITY, 0.f, 0x7fffffff};
    if (active) {
        const int j = b / cpr;
        const int c = b - j * cpr;
        const int slot = __builtin_ctzll(__builtin_amdgcn_ballot_w64(in_mask && rank == j));
        const float *x = p.logits + (ob + slot) * (size_t)p.V;
        if ((p.V & 3) == 0) {
            const int V4 = p.V >> 2;
            const int beg = (int)((long long)V4 * c / cpr);
            const int end = (int)((long long)V4 * (c + 1) / cpr);
            const float4 *x4 = reinterpret_cast<const float4 *>(x);
            // Two batches of kBatch / 2 loads per thread alternate: the next
            // batch is in flight while the current one is reduced.  Each logit
            // is read once, so the loads are non-temporal.
            constexpr int HB = kBatch / 2;
            constexpr int STEP = NT * HB;
            float4 va[HB], vb[HB];
            auto load = [&](float4(&v)[HB], int u0) __attribute__((always_inline)) {
#pragma unroll
                for (int k = 0; k < HB; ++k) {
                    const int u = u0 + k * NT + tid;
                    if (u < end) {
                        const floatx4 t = __builtin_nontemporal_load(reinterpret_cast<const floatx4 *>(x4) + u);
                        v[k] = make_float4(t[0], t[1], t[2], t[3]);
                    }
                }
            };
            auto reduce = [&](const float4(&v)[HB], int u0) __attribute__((always_inline)) {
#pragma unroll
                for (int k = 0; k < HB; ++k) {
                    const int u = u0 + k * NT + tid;
                    if (u < end) push4<!VERIFY>(acc, v[k], 4 * u);
                }
            };
            load(va, beg);
            for (int u0 = beg; u0 < end; u0 += 2 * STEP) {
                if (u0 + STEP < end) load(vb, u0 + STEP);
                reduce(va, u0);
                if (u0 + 2 * STEP < end) load(va, u0 + 2 * STEP);
                if (u0 + STEP < end) reduce(vb, u0 + STEP);
            }
        } else {
            const int beg = (int)((long long)p.V * c / cpr);
            const int end = (int)((long long)p.V * (c + 1) / cpr);
            for (int e0 = beg; e0 < end; e0 += NT * kBatch) {
                float v[kBatch];
#pragma unroll
                for (int k = 0; k < kBatch; ++k) {
                    const int e = e0 + k * NT + tid;
                    if (e < end) v[k] = __builtin_nontemporal_load(x + e);
                }
#pragma unroll
                for (int k = 0; k < kBatch; ++k) {
                    const int e = e0 + k * NT + tid;
                    if (e < end) push<!VERIFY>(acc, v[k], e);
                }
            }
        }
    }
    acc = wave_reduce(acc);
    if (lane == 0) s_part[w] = acc;
    __syncthreads();
    if (tid == 0) {
        // Publish: every workgroup, idle ones included (an idle partial is the
        // identity), writes its slot only after its flag reads have returned
        // (the partial depends on them).  Each word is one 64-bit atomic store
        // whose upper half is non-zero, so a reader that sees it non-zero sees
        // the whole word of this call.
        Part t = s_part[0];
#pragma unroll
        for (int k = 1; k < NT / 64; ++k) t = combine(t, s_part[k]);
        uint64_t *slot = p.part + ((size_t)r * p.G + b) * 2;
        bd_coherent_store64(slot, ((uint64_t)((uint32_t)t.i + 2u) << 32) | __float_as_uint(t.m));
        bd_coherent_store64(slot + 1, (1ull << 32) | __float_as_uint(t.s));
        s_done = tk == gsize - 1 && (p.NG == 1 || rq == p.NG - 1);
    }
    __syncthreads();
    if (!s_done) return;

    // Finisher of request r.  Every ticket is taken: reset the request counter.
    // Then wait until all G slots are published (which also means every
    // workgroup has read the masked flags rewritten below) and stage the
    // nm * cpr partials (chunk c of row j at j * cpr + c) in LDS.  The wait is
    // bounded so the kernel always ends; it cannot run out, since every
    // workgroup of the request has started and publishes without waiting.
    if (tid == 0 && p.NG > 1) bd_coherent_store(rc, 0);
    const int n_part = nm * cpr;
    {
        uint64_t *pp = p.part + (size_t)r * p.G * 2;
        constexpr int PER = kMaxGroups / NT;
        uint64_t wa[PER], wb[PER];
        unsigned pend = 0;
#pragma unroll
        for (int k = 0; k < PER; ++k) {
            wa[k] = wb[k] = 0;
            if (tid + k * NT < p.G) pend |= 1u << k;
        }
        for (int it = 0; pend != 0 && it < kPollLimit; ++it) {
#pragma unroll
            for (int k = 0; k < PER; ++k)
                if ((pend >> k) & 1u) {
                    const int q = tid + k * NT;
                    wa[k] = bd_coherent_load64(pp + 2 * q);
                    wb[k] = bd_coherent_load64(pp + 2 * q + 1);
                }
#pragma unroll
            for (int k = 0; k < PER; ++k)
                if ((wa[k] >> 32) != 0 && (wb[k] >> 32) != 0) pend &= ~(1u << k);
            if (pend != 0) __builtin_amdgcn_s_sleep(1);
        }
#pragma unroll
        for (int k = 0; k < PER; ++k) {
            const int q = tid + k * NT;
            if (q < n_part) {
                s_ms[q] = make_float2(__uint_as_float((uint32_t)wa[k]), __uint_as_float((uint32_t)wb[k]));
                s_i[q] = (int)((uint32_t)(wa[k] >> 32) - 2u);
            }
            if (q < p.G) {  // read: clear the slot for the next call
                bd_coherent_store64(pp + 2 * q, 0);
                bd_coherent_store64(pp + 2 * q + 1, 0);
            }
        }
    }
    if (w == 0 && in_mask) s_slot[rank] = lane;
    __syncthreads();
    // Sixteen lanes per row: lane c takes chunks c, c + 16, ... in order, then a
    // fixed 16-lane tree; sixteen rows per pass.
    for (int j0 = 0; j0 < nm; j0 += NT / 16) {
        const int j = j0 + (tid >> 4);
        const int c0 = tid & 15;
        Part t{-INFINITY, 0.f, 0x7fffffff};
        if (j < nm) {
            // Four chunks' partials are read before they are combined (in
            // chunk order), so the LDS latency is paid once per four.
            int c = c0;
            for (; c + 48 < cpr; c += 64) {
                float2 m2[4];
                int ix[4];
#pragma unroll
                for (int u = 0; u < 4; ++u) {
                    m2[u] = s_ms[j * cpr + c + 16 * u];
                    ix[u] = s_i[j * cpr + c + 16 * u];
                }
#pragma unroll
                for (int u = 0; u < 4; ++u) t = combine(t, Part{m2[u].x, m2[u].y, ix[u]});
            }
            for (; c < cpr; c += 16) {
                const float2 m2 = s_ms[j * cpr + c];
                t = combine(t, Part{m2.x, m2.y, s_i[j * cpr + c]});
            }
        }
        t = reduce16(t);
        if (j < nm && c0 == 0) {
            const int slot = s_slot[j];
            s_conf[slot] = 1.0f / t.s;
            s_arg[slot] = t.i;
        }
    }
    __syncthreads();
    if (w != 0) return;
    if (VERIFY) {
        const int a = lane < p.D ? s_arg[lane] : 0;
        const bool bad = lane < p.D && a != p.draft[ob + lane];
        const unsigned long long bb = __builtin_amdgcn_ballot_w64(bad);
        if (lane < p.D && p.argmax) p.argmax[ob + lane] = a;
        if (lane == 0) p.accepted_len[r] = bb ? (__ffsll((long long)bb) - 1) : p.D;
        return;
    }
    const unsigned long long tb = commit_request(s_conf, s_arg, mask, nm, p.D, p.S, p.tau, lane, p.masked + ob,
                                                 p.tokens + ob, p.conf ? p.conf + ob : nullptr,
                                                 p.argmax ? p.argmax + ob : nullptr,
                                                 p.committed ? p.committed + ob : nullptr);
    if (lane == 0 && p.n_committed) p.n_committed[r] = __popcll(tb);
}

RowParams make_params(const RowPlan &pl, const RowArgs &a) {
    RowParams p{};
    p.logits = a.logits;
    p.masked = a.masked;
    p.tokens = a.tokens;
    p.conf = a.conf;
    p.argmax = a.argmax;
    p.committed = a.committed;
    p.n_committed = a.n_committed;
    p.draft = a.draft;
    p.accepted_len = a.accepted_len;
    char *ws = (char *)a.ws;
    p.part = (uint64_t *)(ws + pl.part_off);
    p.grp_cnt = (int *)(ws + pl.grp_off);
    p.req_cnt = (int *)(ws + pl.cnt_off);
    p.n_req = a.n_req;
    p.D = a.D;
    p.V = a.V;
    p.S = a.S;
    p.G = pl.groups;
    p.NG = (pl.groups + kTicketGroup - 1) / kTicketGroup;
    p.max_cpr = pl.max_cpr;
    p.tau = a.tau;
    return p;
}

}  // namespace

RowPlan plan_rows(int n_req, int D, int V) {
    RowPlan pl{};
    // Chunks per row if every slot took part: enough workgroups for the call to
    // fill the GPU (kWgTarget), no chunk above kMaxChunk floats where the rows
    // allow, none below kMinChunk, and at most kMaxGroups workgroups per request.
    const long long c_lo = ((long long)V + kMaxChunk - 1) / kMaxChunk;
    const long long c_hi = std::max(1ll, ((long long)V + kMinChunk - 1) / kMinChunk);
    const long long c_want = ((long long)kWgTarget + (long long)n_req * D - 1) / ((long long)n_req * D);
    long long c0 = std::min(std::max(c_want, c_lo), c_hi);
    c0 = std::max(1ll, std::min(c0, (long long)(kMaxGroups / D)));
    pl.groups = (int)(D * c0);
    pl.max_cpr = std::max((int)c0, V / kMinChunkRun);
    pl.ok = (long long)n_req * pl.groups * NT < (1ll << 32);  // HIP grid limit
    size_t off = 0;
    auto take = [&](size_t bytes) {
        size_t o = off;
        off += (bytes + 255) / 256 * 256;
        return o;
    };
    pl.part_off = take((size_t)n_req * pl.groups * 16);
    const int ng = (pl.groups + kTicketGroup - 1) / kTicketGroup;
    pl.grp_off = take((size_t)n_req * ng * kCounterStride * 4);
    pl.cnt_off = take((size_t)n_req * kCounterStride * 4);
    pl.ws_bytes = off;
    return pl;
}

hipError_t launch_confidence_commit(const RowPlan &pl, const RowArgs &a, hipStream_t s) {
    RowParams p = make_params(pl, a);
    hipLaunchKernelGGL((row_kernel<false>), dim3(a.n_req * pl.groups), dim3(NT), 0, s, p);
    return hipGetLastError();
}

hipError_t launch_spec_verify(const RowPlan &pl, const RowArgs &a, hipStream_t s) {
    RowParams p = make_params(pl, a);
    hipLaunchKernelGGL((row_kernel<true>), dim3(a.n_req * pl.groups), dim3(NT), 0, s, p);
    return hipGetLastError();
}

// ---------------------------------------------------------------------------
// KV append (Fast-dVLM write-up, section 5.3: crop the cache to the accepted
// prefix; DiffusionVL notes: a finished block joins the history cache).
// One workgroup per item, so the prefix length it reads and advances has a
// single reader and writer; no host round trip is needed between verify and
// append.  The host bounds S * Hkv * d by 2^30, so unit indices fit 32 bits.
// ---------------------------------------------------------------------------
constexpr int kAppendThreads = 512;

__global__ __launch_bounds__(kAppendThreads) void kv_append_kernel(int D, int S, int Hkv, int row_bytes, int cap,
                                                                   uint8_t *k_cache, uint8_t *v_cache, int32_t *prefix,
                                                                   const uint8_t *k_blk, const uint8_t *v_blk,
                                                                   const int32_t *n_accept, int32_t *dev_err) {
    const int it = blockIdx.x;
    const int P = prefix[it];
    const int L = n_accept ? n_accept[it] : D;
    if (L < 0 || L > D || P < 0 || P + L > cap) {
        if (threadIdx.x == 0 && dev_err) *dev_err = 1;
        return;
    }
    // K and V rows alike: block [slot][Hkv][d] -> cache [Hkv][cap][d], whole
    // 16-byte units (a row is 64 to 512 bytes).  Consecutive threads read
    // consecutive units of the block.
    const int U = row_bytes / 16;
    const int per_t = Hkv * U;
    const int n = L * per_t;  // <= S * Hkv * d * 4 / 16 <= 2^28
    const size_t src0 = (size_t)it * S * per_t;
    for (int e = threadIdx.x; e < n; e += kAppendThreads) {
        const int t = e / per_t, r = e - t * per_t;
        const int g = r / U, u = r - g * U;
        const size_t src = src0 + e;
        const size_t dst = (((size_t)it * Hkv + g) * cap + P + t) * U + u;
        reinterpret_cast<uint4 *>(k_cache)[dst] = reinterpret_cast<const uint4 *>(k_blk)[src];
        reinterpret_cast<uint4 *>(v_cache)[dst] = reinterpret_cast<const uint4 *>(v_blk)[src];
    }
    __syncthreads();  // every thread has read P
    if (threadIdx.x == 0) prefix[it] = P + L;
}

hipError_t launch_kv_append(int n, int D, int S, int Hkv, int d, int cap, int elem_bytes, void *k_cache, void *v_cache,
                            int32_t *prefix, const void *k_blk, const void *v_blk, const int32_t *n_accept,
                            int32_t *dev_err, hipStream_t s) {
    hipLaunchKernelGGL(kv_append_kernel, dim3(n), dim3(kAppendThreads), 0, s, D, S, Hkv, d * elem_bytes, cap,
                       (uint8_t *)k_cache, (uint8_t *)v_cache, prefix, (const uint8_t *)k_blk, (const uint8_t *)v_blk,
                       n_accept, dev_err);
    return hipGetLastError();
}

}  // namespace bd
