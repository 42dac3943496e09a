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
// Each row is split into chunks of whole 1024-float strides; one 256-thread
// workgroup streams one chunk with 16-byte loads, keeping a running
// (max, index of first max, sum of exp(x - max)) per thread.  Partials are
// combined in a fixed tree inside the workgroup; the last workgroup of a
// request (one atomic ticket per request) merges every row's chunk partials
// in chunk order and runs the one-wave commit / verify tail.  No float atomics, so
// results are identical run to run.
#include "bd_common.h"
#include "bd_internal.h"
#include "bd_rowreduce.h"

namespace bd {
namespace {

constexpr int NT = 256;
constexpr int kRowLoads = 16;  // float4 loads per thread per chunk (chunk <= 16 x 1024 floats)

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
    float *part_m, *part_s;
    int *part_i;
    int *req_cnt;
    int n_req, D, V, S, chunks, chunk_elems;
    float tau;
};

template <bool VERIFY>
__global__ __launch_bounds__(NT) void row_kernel(RowParams p) {
    __shared__ Part s_part[NT / 64];
    __shared__ __attribute__((aligned(16))) float s_conf[64];
    __shared__ int s_arg[64];
    __shared__ int s_done, s_nm;
    __shared__ unsigned long long s_mask;
    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int w = tid >> 6;
    const int row = blockIdx.x / p.chunks;
    const int chunk = blockIdx.x - row * p.chunks;
    const int r = row / p.D;
    const int slot = row - r * p.D;
    const size_t ob = (size_t)r * p.D;

    // The masked flags are requested first and the chunk's logits right behind
    // them (all of a thread's loads in flight together), so deciding whether this
    // row takes part costs no extra round trip; rows that do not take part drop
    // their loads.
    bool mk = false;
    if (!VERIFY && w == 0) mk = lane < p.D && p.masked[ob + lane] != 0;
    const float *x = p.logits + (size_t)row * p.V;
    const int beg = chunk * p.chunk_elems;
    const int end = min(p.V, beg + p.chunk_elems);
    const bool vec = (p.V & 3) == 0;
    float4 v[kRowLoads];
    if (vec) {
#pragma unroll
        for (int u = 0; u < kRowLoads; ++u) {
            const int e = beg + tid * 4 + u * NT * 4;
            if (e < end) v[u] = *reinterpret_cast<const float4 *>(x + e);
        }
    }
    if (!VERIFY) {
        if (w == 0) {
            const unsigned long long b = __builtin_amdgcn_ballot_w64(mk);
            if (lane == 0) {
                s_mask = b;
                s_nm = __popcll(b);
            }
        }
        __syncthreads();
        if (!((s_mask >> slot) & 1ull)) {
            // A request with nothing masked still reports an empty commit.
            if (s_nm == 0 && slot == 0 && chunk == 0 && w == 0 && lane < p.D) {
                if (p.conf) p.conf[ob + lane] = __int_as_float(0x7fc00000);
                if (p.argmax) p.argmax[ob + lane] = -1;
                if (p.committed) p.committed[ob + lane] = 0;
                if (p.n_committed && lane == 0) p.n_committed[r] = 0;
            }
            return;
        }
    }

    // Reduce this chunk of the row.
    Part acc{-INFINITY, 0.f, 0x7fffffff};
    if (vec) {
#pragma unroll
        for (int u = 0; u < kRowLoads; ++u) {
            const int e = beg + tid * 4 + u * NT * 4;
            if (e < end) {
                push<!VERIFY>(acc, v[u].x, e);
                push<!VERIFY>(acc, v[u].y, e + 1);
                push<!VERIFY>(acc, v[u].z, e + 2);
                push<!VERIFY>(acc, v[u].w, e + 3);
            }
        }
    } else {
        for (int e = beg + tid; e < end; e += NT) push<!VERIFY>(acc, x[e], e);
    }
    acc = wave_reduce(acc);
    if (lane == 0) s_part[w] = acc;
    __syncthreads();
    if (tid == 0) {
        Part t = s_part[0];
#pragma unroll
        for (int k = 1; k < NT / 64; ++k) t = combine(t, s_part[k]);
        const size_t o = (size_t)row * p.chunks + chunk;
        bd_coherent_store(p.part_m + o, t.m);
        bd_coherent_store(p.part_s + o, t.s);
        bd_coherent_store(p.part_i + o, t.i);
        bd_wait_all_memory();
        // One ticket per request: the last of its (rows x chunks) workgroups finishes it.
        const int need = (VERIFY ? p.D : s_nm) * p.chunks;
        s_done = bd_ticket(&p.req_cnt[r]) == need - 1;
    }
    __syncthreads();
    if (!s_done) return;

    // Last workgroup of request r.  Sixteen lanes per row merge that row's chunk
    // partials (lane c takes chunks c, c + 16, ... in order, then a fixed
    // 16-lane tree), four rows per wave, sixteen rows per pass.
    for (int r0 = 0; r0 < p.D; r0 += 16) {
        const int i = r0 + w * 4 + (lane >> 4);
        const bool act = i < p.D && (VERIFY || ((s_mask >> i) & 1ull));
        Part t{-INFINITY, 0.f, 0x7fffffff};
        if (act) {
            const size_t o = (ob + i) * p.chunks;
            for (int c = lane & 15; c < p.chunks; c += 16)
                t = combine(t, Part{bd_coherent_load(p.part_m + o + c), bd_coherent_load(p.part_s + o + c),
                                    bd_coherent_load(p.part_i + o + c)});
        }
        t = reduce16(t);
        if (act && (lane & 15) == 0) {
            s_conf[i] = 1.0f / t.s;
            s_arg[i] = t.i;
        }
    }
    __syncthreads();
    if (w != 0) return;
    if (VERIFY) {
        const int a = lane < p.D ? s_arg[lane] : 0;
        const bool bad = lane < p.D && a != p.draft[ob + lane];
        const unsigned long long b = __builtin_amdgcn_ballot_w64(bad);
        if (lane < p.D && p.argmax) p.argmax[ob + lane] = a;
        if (lane == 0) {
            p.accepted_len[r] = b ? (__ffsll((long long)b) - 1) : p.D;
            bd_coherent_store(p.req_cnt + r, 0);
        }
        return;
    }
    const unsigned long long tb = commit_request(s_conf, s_arg, s_mask, s_nm, p.D, p.S, p.tau, lane, p.masked + ob,
                                                 p.tokens + ob, p.conf ? p.conf + ob : nullptr,
                                                 p.argmax ? p.argmax + ob : nullptr,
                                                 p.committed ? p.committed + ob : nullptr);
    if (lane == 0) {
        if (p.n_committed) p.n_committed[r] = __popcll(tb);
        bd_coherent_store(p.req_cnt + r, 0);
    }
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
    const size_t np = (size_t)pl.rows * pl.chunks;
    p.part_m = (float *)(ws + pl.part_off);
    p.part_s = p.part_m + np;
    p.part_i = (int *)(p.part_s + np);
    p.req_cnt = (int *)(ws + pl.cnt_off);
    p.n_req = a.n_req;
    p.D = a.D;
    p.V = a.V;
    p.S = a.S;
    p.chunks = pl.chunks;
    p.chunk_elems = pl.chunk_elems;
    p.tau = a.tau;
    return p;
}

}  // namespace

RowPlan plan_rows(int n_req, int D, int V) {
    RowPlan pl{};
    pl.rows = n_req * D;
    // Chunks of about 16 strides of 1024 floats (64 KB): enough bytes per
    // workgroup to keep its loads streaming, few enough workgroups per request
    // that its ticket counter is not a point of contention.  Rows that are
    // short or few get smaller chunks so that at least ~256 workgroups run.
    const int strides = (V + 1023) / 1024;  // 1024-float strides per row
    int chunks = std::max(1, (strides + 15) / 16);
    const int want = std::max(1, (256 + pl.rows - 1) / pl.rows);
    chunks = std::min(strides, std::max(chunks, want));
    const int per = (strides + chunks - 1) / chunks;
    pl.chunk_elems = per * 1024;
    pl.chunks = (V + pl.chunk_elems - 1) / pl.chunk_elems;
    pl.ok = (size_t)pl.rows * pl.chunks * NT < (1ull << 32);  // HIP grid limit
    size_t off = 0;
    auto take = [&](size_t bytes) {
        size_t o = off;
        off += (bytes + 255) / 256 * 256;
        return o;
    };
    pl.part_off = take((size_t)pl.rows * pl.chunks * 12);
    pl.cnt_off = take((size_t)n_req * 4);
    pl.ws_bytes = off;
    return pl;
}

hipError_t launch_confidence_commit(const RowPlan &pl, const RowArgs &a, hipStream_t s) {
    RowParams p = make_params(pl, a);
    hipLaunchKernelGGL((row_kernel<false>), dim3(pl.rows * pl.chunks), dim3(NT), 0, s, p);
    return hipGetLastError();
}

hipError_t launch_spec_verify(const RowPlan &pl, const RowArgs &a, hipStream_t s) {
    RowParams p = make_params(pl, a);
    hipLaunchKernelGGL((row_kernel<true>), dim3(pl.rows * pl.chunks), dim3(NT), 0, s, p);
    return hipGetLastError();
}

// ---------------------------------------------------------------------------
// KV append (Fast-dVLM write-up, section 5.3: crop the cache to the accepted
// prefix; DiffusionVL notes: a finished block joins the history cache).
// One workgroup per item; the prefix length is read on the device, so no
// host round trip is needed between verify and append.
// ---------------------------------------------------------------------------
template <typename E>
__global__ __launch_bounds__(256) void kv_append_kernel(int D, int S, int Hkv, int d, int cap, E *k_cache, E *v_cache,
                                                        int32_t *prefix, const E *k_blk, const E *v_blk,
                                                        const int32_t *n_accept, int32_t *dev_err) {
    const int it = blockIdx.x;
    const int P = prefix[it];
    const int L = n_accept ? n_accept[it] : D;
    if (L < 0 || L > D || P < 0 || P + L > cap) {
        if (threadIdx.x == 0 && dev_err) *dev_err = 1;
        return;
    }
    const int per_t = Hkv * d;
    for (int e = threadIdx.x; e < L * per_t; e += blockDim.x) {
        const int t = e / per_t;
        const int g = (e / d) % Hkv;
        const int dd = e % d;
        const size_t src = (((size_t)it * S + t) * Hkv + g) * d + dd;
        k_cache[(((size_t)it * Hkv + g) * cap + (P + t)) * d + dd] = k_blk[src];
        v_cache[(((size_t)it * Hkv + g) * d + dd) * cap + (P + t)] = v_blk[src];
    }
    __syncthreads();
    if (threadIdx.x == 0) prefix[it] = P + L;
}

hipError_t launch_kv_append(int n, int D, int S, int Hkv, int d, int cap, int elem_bytes, void *k_cache, void *v_cache,
                            int32_t *prefix, const void *k_blk, const void *v_blk, const int32_t *n_accept,
                            int32_t *dev_err, hipStream_t s) {
    if (elem_bytes == 4)
        hipLaunchKernelGGL((kv_append_kernel<uint32_t>), dim3(n), dim3(256), 0, s, D, S, Hkv, d, cap,
                           (uint32_t *)k_cache, (uint32_t *)v_cache, prefix, (const uint32_t *)k_blk,
                           (const uint32_t *)v_blk, n_accept, dev_err);
    else if (elem_bytes == 2)
        hipLaunchKernelGGL((kv_append_kernel<uint16_t>), dim3(n), dim3(256), 0, s, D, S, Hkv, d, cap,
                           (uint16_t *)k_cache, (uint16_t *)v_cache, prefix, (const uint16_t *)k_blk,
                           (const uint16_t *)v_blk, n_accept, dev_err);
    else
        hipLaunchKernelGGL((kv_append_kernel<uint8_t>), dim3(n), dim3(256), 0, s, D, S, Hkv, d, cap,
                           (uint8_t *)k_cache, (uint8_t *)v_cache, prefix, (const uint8_t *)k_blk,
                           (const uint8_t *)v_blk, n_accept, dev_err);
    return hipGetLastError();
}

}  // namespace bd
