// C-ABI entry points of libbd: host-side validation, workspace sizing and launch.
// Every check runs before any HIP call, so invalid arguments are reported
// without touching the device (and can be exercised on a machine without a GPU).
#include <math.h>
#include <stdint.h>

#include <algorithm>
#include <mutex>

#include "../../include/bd.h"
#include "bd_internal.h"

// Fixed device memory of bd_attn_step_noalloc: the split-K exchange of one
// call at a time per GPU.  Every GPU the library runs on holds its own copy
// (64 MiB) until the process ends.
static __device__ __align__(256) unsigned char scratch[BD_NOALLOC_SCRATCH_BYTES];

namespace {

thread_local int32_t g_last_hip_error = 0;

bool aligned16(const void *p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

// The mask mode without the plan flag.
int mask_mode(const bd_attn_desc *d) { return d->mode & ~BD_PLAN_BALANCED; }
bool balanced_hint(const bd_attn_desc *d) { return (d->mode & BD_PLAN_BALANCED) != 0; }

// Block slots per item: D, or B (B + 3) / 2 for the quadratic mode (D = B).
int block_slots(const bd_attn_desc *d) { return mask_mode(d) == BD_BLOCK_QUAD ? d->D * (d->D + 3) / 2 : d->D; }

// Launch sizes stay within 32-bit grid and index arithmetic: at most
// kMaxSplits workgroups per (item, KV head, 128-row block) on the MFMA path,
// one wave per query row on the vector path.  Called once slots * Hq <= 2^20.
bool launch_fits(int64_t n, int64_t slots, int64_t Hq, int64_t Hkv) {
    const int64_t row_blocks = (slots * (Hq / Hkv) + 127) / 128;
    int64_t units = 0, rows = 0;
    if (__builtin_mul_overflow(n, Hkv * row_blocks, &units) || units > INT32_MAX / bd::kMaxSplits - 1) return false;
    if (__builtin_mul_overflow(n, slots * Hq, &rows) || rows / 4 >= INT32_MAX) return false;
    return true;
}

bd_status check_attn_desc(const bd_attn_desc *d) {
    if (!d) return BD_E_NULL;
    if (d->dtype != BD_F32 && d->dtype != BD_BF16 && d->dtype != BD_FP8KV) return BD_E_DTYPE;
    const int m = mask_mode(d);
    if (m != BD_BLOCK_BIDIR && m != BD_BLOCK_CAUSAL && m != BD_BLOCK_QUAD) return BD_E_PARAM;
    if (!(d->scale > 0.f) || !isfinite(d->scale)) return BD_E_PARAM;
    if (d->n_items < 1 || d->D < 1 || d->D > (m == BD_BLOCK_QUAD ? 32 : 64)) return BD_E_SHAPE;
    if (d->Hq < 1 || d->Hkv < 1 || d->Hq % d->Hkv != 0) return BD_E_SHAPE;
    if (d->d != 64 && d->d != 128) return BD_E_SHAPE;
    if (d->cap < 1) return BD_E_SHAPE;
    if (d->max_prefix < 0 || d->max_prefix > d->cap) return BD_E_SHAPE;
    // Index arithmetic in the kernels uses 32-bit ints for per-item quantities.
    if ((int64_t)block_slots(d) * d->Hq > (1 << 20) || (int64_t)d->cap * d->d > (1ll << 30)) return BD_E_SHAPE;
    if (!launch_fits(d->n_items, block_slots(d), d->Hq, d->Hkv)) return BD_E_SHAPE;
    return BD_OK;
}

bd_status check_commit_desc(const bd_commit_desc *d) {
    if (!d) return BD_E_NULL;
    if (d->n_req < 1 || d->D < 1 || d->D > 64 || d->V < 2) return BD_E_SHAPE;
    if ((int64_t)d->n_req * d->D > (1 << 24)) return BD_E_SHAPE;
    if (d->S < 1 || isnan(d->tau)) return BD_E_PARAM;
    return BD_OK;
}

bd_status check_rows(int32_t n_req, int32_t D, int32_t V) {
    if (n_req < 1 || D < 1 || D > 64 || V < 2) return BD_E_SHAPE;
    if ((int64_t)n_req * D > (1 << 24)) return BD_E_SHAPE;
    return BD_OK;
}

bd_status check_lmhead_desc(const bd_lmhead_desc *d) {
    if (!d) return BD_E_NULL;
    if (d->n_req < 1 || d->D < 1 || d->D > 64 || (int64_t)d->n_req * d->D > 16) return BD_E_SHAPE;
    if (d->V < 2 || d->H < 256 || d->H % 256 != 0 || d->H > 4096) return BD_E_SHAPE;
    if (d->S < 1 || isnan(d->tau)) return BD_E_PARAM;
    return BD_OK;
}

bd_status check_two_stream_desc(const bd_two_stream_desc *d) {
    if (!d) return BD_E_NULL;
    if (!(d->scale > 0.f) || !isfinite(d->scale)) return BD_E_PARAM;
    if (d->n_seq < 1 || d->Lc < 1 || d->Ln < 0 || d->D < 1 || d->D > 4096) return BD_E_SHAPE;
    if (d->Hq < 1 || d->Hkv < 1 || d->Hq % d->Hkv != 0) return BD_E_SHAPE;
    if (d->d != 64 && d->d != 128) return BD_E_SHAPE;
    const int64_t L = (int64_t)d->Lc + d->Ln;
    if (d->cap < L || d->cap % 32 != 0) return BD_E_SHAPE;
    if (d->max_spans < 0 || d->max_spans > 256 || (d->Ln > 0 && d->max_spans < 1)) return BD_E_SHAPE;
    if (L * d->Hq > (1 << 20) || (int64_t)d->cap * d->d > (1ll << 30)) return BD_E_SHAPE;
    if (!launch_fits(d->n_seq, L, d->Hq, d->Hkv)) return BD_E_SHAPE;
    return BD_OK;
}

bd_status launched(hipError_t e) {
    if (e != hipSuccess) {
        g_last_hip_error = (int32_t)e;
        return BD_E_LAUNCH;
    }
    return BD_OK;
}

// Device address of the current device's copy of `scratch`, looked up once per
// device.  In host code `scratch` names a host-side stand-in; only this address
// may be handed to kernels.
constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void *g_scratch_ptr[kMaxDevices] = {};

hipError_t scratch_address(hipStream_t stream, void **out) {
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return e;
    if (stream) {
        hipDevice_t sdev = 0;
        e = hipStreamGetDevice(stream, &sdev);
        if (e != hipSuccess) return e;
        if (sdev != dev) return hipErrorInvalidDevice;  // the stream must belong to the current device
    }
    if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
    std::lock_guard<std::mutex> lock(g_scratch_mu);
    if (!g_scratch_ptr[dev]) {
        void *ptr = nullptr;
        e = hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch));
        if (e != hipSuccess) return e;
        g_scratch_ptr[dev] = ptr;
    }
    *out = g_scratch_ptr[dev];
    return hipSuccess;
}

}  // namespace

extern "C" {

size_t bd_attn_workspace_bytes(const bd_attn_desc *desc) {
    if (check_attn_desc(desc) != BD_OK) return SIZE_MAX;
    const bd::AttnPlan pl = bd::plan_attention(desc->n_items, block_slots(desc), desc->Hq, desc->Hkv, desc->d,
                                               desc->dtype, desc->max_prefix, false, balanced_hint(desc));
    return pl.ws_bytes;
}

namespace {
bd_status attn_common(const bd_attn_desc *desc, const void *q, const void *k_blk, const void *v_blk,
                      const void *k_cache, const void *v_cache, const float *k_scale, const float *v_scale,
                      const int32_t *prefix_len, void *out, void *workspace, size_t workspace_bytes,
                      void *stream) {
    const bd::AttnPlan pl = bd::plan_attention(desc->n_items, block_slots(desc), desc->Hq, desc->Hkv, desc->d,
                                               desc->dtype, desc->max_prefix, false, balanced_hint(desc));
    if (pl.ws_bytes > 0 && (!workspace || workspace_bytes < pl.ws_bytes || !aligned16(workspace)))
        return BD_E_WORKSPACE;
    bd::AttnArgs a{};
    a.q = q;
    a.k_blk = k_blk;
    a.v_blk = v_blk;
    a.k_cache = k_cache;
    a.v_cache = v_cache;
    a.prefix = prefix_len;
    a.k_scale = k_scale;
    a.v_scale = v_scale;
    a.out = out;
    a.ws = workspace;
    a.n = desc->n_items;
    a.D = block_slots(desc);
    a.B = mask_mode(desc) == BD_BLOCK_QUAD ? desc->D : 0;
    a.Hq = desc->Hq;
    a.Hkv = desc->Hkv;
    a.d = desc->d;
    a.cap = desc->cap;
    a.mode = mask_mode(desc);
    a.scale = desc->scale;
    hipStream_t s = (hipStream_t)stream;
    return launched(pl.mfma ? bd::launch_attention_mfma(pl, a, s) : bd::launch_attention_vec(a, desc->dtype, s));
}
}  // namespace

bd_status bd_attn_step(const bd_attn_desc *desc, const void *q, const void *k_blk, const void *v_blk,
                       const void *k_cache, const void *v_cache, const int32_t *prefix_len, void *out,
                       void *workspace, size_t workspace_bytes, void *stream) {
    bd_status st = check_attn_desc(desc);
    if (st != BD_OK) return st;
    if (desc->dtype == BD_FP8KV) return BD_E_DTYPE;  // needs the scales: bd_attn_step_fp8kv
    if (!q || !k_blk || !v_blk || !k_cache || !v_cache || !prefix_len || !out) return BD_E_NULL;
    if (!aligned16(q) || !aligned16(k_blk) || !aligned16(v_blk) || !aligned16(k_cache) ||
        !aligned16(v_cache) || !aligned16(out))
        return BD_E_PARAM;
    return attn_common(desc, q, k_blk, v_blk, k_cache, v_cache, nullptr, nullptr, prefix_len, out, workspace,
                       workspace_bytes, stream);
}

bd_status bd_attn_step_noalloc(const bd_attn_desc *desc, const void *q, const void *k_blk, const void *v_blk,
                               const void *k_cache, const void *v_cache, const int32_t *prefix_len, void *out,
                               void *stream) {
    bd_status st = check_attn_desc(desc);
    if (st != BD_OK) return st;
    if (desc->dtype == BD_FP8KV) return BD_E_DTYPE;
    if (!q || !k_blk || !v_blk || !k_cache || !v_cache || !prefix_len || !out) return BD_E_NULL;
    if (!aligned16(q) || !aligned16(k_blk) || !aligned16(v_blk) || !aligned16(k_cache) ||
        !aligned16(v_cache) || !aligned16(out))
        return BD_E_PARAM;
    const bd::AttnPlan pl = bd::plan_attention(desc->n_items, block_slots(desc), desc->Hq, desc->Hkv, desc->d,
                                               desc->dtype, desc->max_prefix, false, balanced_hint(desc));
    if (pl.ws_bytes > BD_NOALLOC_SCRATCH_BYTES) return BD_E_SCRATCH;
    void *ws = nullptr;
    if (pl.ws_bytes > 0) {
        const hipError_t e = scratch_address((hipStream_t)stream, &ws);
        if (e != hipSuccess) return launched(e);
    }
    return attn_common(desc, q, k_blk, v_blk, k_cache, v_cache, nullptr, nullptr, prefix_len, out, ws,
                       BD_NOALLOC_SCRATCH_BYTES, stream);
}

size_t bd_attn_noalloc_max_scratch_bytes(void) { return BD_NOALLOC_SCRATCH_BYTES; }

bd_status bd_attn_step_fp8kv(const bd_attn_desc *desc, const void *q, const void *k_blk, const void *v_blk,
                             const void *k_cache, const void *v_cache, const float *k_scale,
                             const float *v_scale, const int32_t *prefix_len, void *out, void *workspace,
                             size_t workspace_bytes, void *stream) {
    bd_status st = check_attn_desc(desc);
    if (st != BD_OK) return st;
    if (desc->dtype != BD_FP8KV) return BD_E_DTYPE;
    if (!q || !k_blk || !v_blk || !k_cache || !v_cache || !k_scale || !v_scale || !prefix_len || !out)
        return BD_E_NULL;
    if (!aligned16(q) || !aligned16(k_blk) || !aligned16(v_blk) || !aligned16(k_cache) ||
        !aligned16(v_cache) || !aligned16(out))
        return BD_E_PARAM;
    return attn_common(desc, q, k_blk, v_blk, k_cache, v_cache, k_scale, v_scale, prefix_len, out, workspace,
                       workspace_bytes, stream);
}

size_t bd_commit_workspace_bytes(const bd_commit_desc *desc) {
    if (check_commit_desc(desc) != BD_OK) return SIZE_MAX;
    const bd::RowPlan pl = bd::plan_rows(desc->n_req, desc->D, desc->V);
    return pl.ok ? pl.ws_bytes : SIZE_MAX;
}

bd_status bd_confidence_commit(const bd_commit_desc *desc, const float *logits, uint8_t *masked,
                               int32_t *tokens, float *conf, int32_t *argmax, uint8_t *committed,
                               int32_t *n_committed, void *workspace, size_t workspace_bytes, void *stream) {
    bd_status st = check_commit_desc(desc);
    if (st != BD_OK) return st;
    if (!logits || !masked || !tokens) return BD_E_NULL;
    if (!aligned16(logits)) return BD_E_PARAM;
    const bd::RowPlan pl = bd::plan_rows(desc->n_req, desc->D, desc->V);
    if (!pl.ok) return BD_E_SHAPE;
    if (!workspace || workspace_bytes < pl.ws_bytes || !aligned16(workspace)) return BD_E_WORKSPACE;
    bd::RowArgs a{};
    a.logits = logits;
    a.masked = masked;
    a.tokens = tokens;
    a.conf = conf;
    a.argmax = argmax;
    a.committed = committed;
    a.n_committed = n_committed;
    a.ws = workspace;
    a.n_req = desc->n_req;
    a.D = desc->D;
    a.V = desc->V;
    a.S = desc->S;
    a.tau = desc->tau;
    return launched(bd::launch_confidence_commit(pl, a, (hipStream_t)stream));
}

size_t bd_verify_workspace_bytes(int32_t n_req, int32_t D, int32_t V) {
    if (check_rows(n_req, D, V) != BD_OK) return SIZE_MAX;
    const bd::RowPlan pl = bd::plan_rows(n_req, D, V);
    return pl.ok ? pl.ws_bytes : SIZE_MAX;
}

bd_status bd_spec_verify(int32_t n_req, int32_t D, int32_t V, const float *logits, const int32_t *draft,
                         int32_t *accepted_len, int32_t *argmax, void *workspace, size_t workspace_bytes,
                         void *stream) {
    bd_status st = check_rows(n_req, D, V);
    if (st != BD_OK) return st;
    if (!logits || !draft || !accepted_len) return BD_E_NULL;
    if (!aligned16(logits)) return BD_E_PARAM;
    const bd::RowPlan pl = bd::plan_rows(n_req, D, V);
    if (!pl.ok) return BD_E_SHAPE;
    if (!workspace || workspace_bytes < pl.ws_bytes || !aligned16(workspace)) return BD_E_WORKSPACE;
    bd::RowArgs a{};
    a.logits = logits;
    a.draft = draft;
    a.accepted_len = accepted_len;
    a.argmax = argmax;
    a.ws = workspace;
    a.n_req = n_req;
    a.D = D;
    a.V = V;
    a.S = 1;
    return launched(bd::launch_spec_verify(pl, a, (hipStream_t)stream));
}

bd_status bd_kv_append(const bd_attn_desc *desc, void *k_cache, void *v_cache, int32_t *prefix_len,
                       const void *k_blk, const void *v_blk, const int32_t *n_accept, int32_t *dev_err,
                       void *stream) {
    if (!desc) return BD_E_NULL;
    if (desc->dtype != BD_F32 && desc->dtype != BD_BF16 && desc->dtype != BD_FP8KV) return BD_E_DTYPE;
    const int m = mask_mode(desc);
    if (m != BD_BLOCK_BIDIR && m != BD_BLOCK_CAUSAL && m != BD_BLOCK_QUAD) return BD_E_PARAM;
    if (desc->n_items < 1 || desc->D < 1 || desc->D > (m == BD_BLOCK_QUAD ? 32 : 64) || desc->Hkv < 1)
        return BD_E_SHAPE;
    if (desc->d != 64 && desc->d != 128) return BD_E_SHAPE;
    if (desc->cap < 1) return BD_E_SHAPE;
    // The limits bd_attn_step puts on a cache and a block: one item's cache and
    // one item's block K (or V) hold at most 2^30 elements.
    if ((int64_t)desc->cap * desc->d > (1ll << 30)) return BD_E_SHAPE;
    if ((int64_t)block_slots(desc) * desc->Hkv * desc->d > (1ll << 30)) return BD_E_SHAPE;
    if (!k_cache || !v_cache || !prefix_len || !k_blk || !v_blk) return BD_E_NULL;
    // Rows are copied as 16-byte units.
    if (!aligned16(k_cache) || !aligned16(v_cache) || !aligned16(k_blk) || !aligned16(v_blk)) return BD_E_PARAM;
    // Quadratic mode: the block holds B (B + 3) / 2 slots, of which the first B
    // (the drafts) can be accepted.
    return launched(bd::launch_kv_append(desc->n_items, desc->D, block_slots(desc), desc->Hkv, desc->d, desc->cap,
                                         desc->dtype == BD_F32 ? 4 : desc->dtype == BD_BF16 ? 2 : 1, k_cache,
                                         v_cache, prefix_len, k_blk, v_blk, n_accept, dev_err, (hipStream_t)stream));
}

size_t bd_lmhead_workspace_bytes(const bd_lmhead_desc *desc) {
    if (check_lmhead_desc(desc) != BD_OK) return SIZE_MAX;
    const bd::LhPlan pl = bd::plan_lmhead(desc->n_req, desc->D, desc->V, desc->H);
    return pl.ok ? pl.ws_bytes : SIZE_MAX;
}

bd_status bd_lmhead_confidence_commit(const bd_lmhead_desc *desc, const void *hidden, const void *weight,
                                      uint8_t *masked, int32_t *tokens, float *conf, int32_t *argmax,
                                      uint8_t *committed, int32_t *n_committed, void *workspace,
                                      size_t workspace_bytes, void *stream) {
    bd_status st = check_lmhead_desc(desc);
    if (st != BD_OK) return st;
    if (!hidden || !weight || !masked || !tokens) return BD_E_NULL;
    if (!aligned16(hidden) || !aligned16(weight)) return BD_E_PARAM;
    const bd::LhPlan pl = bd::plan_lmhead(desc->n_req, desc->D, desc->V, desc->H);
    if (!pl.ok) return BD_E_SHAPE;
    if (!workspace || workspace_bytes < pl.ws_bytes || !aligned16(workspace)) return BD_E_WORKSPACE;
    bd::LhArgs a{};
    a.hidden = hidden;
    a.weight = weight;
    a.masked = masked;
    a.tokens = tokens;
    a.conf = conf;
    a.argmax = argmax;
    a.committed = committed;
    a.n_committed = n_committed;
    a.ws = workspace;
    a.n_req = desc->n_req;
    a.D = desc->D;
    a.V = desc->V;
    a.H = desc->H;
    a.S = desc->S;
    a.tau = desc->tau;
    return launched(bd::launch_lmhead(pl, a, (hipStream_t)stream));
}

const char *bd_status_string(bd_status s) {
    switch (s) {
        case BD_OK: return "ok";
        case BD_E_NULL: return "a required pointer is NULL";
        case BD_E_SHAPE: return "a size is out of range or inconsistent";
        case BD_E_DTYPE: return "unknown or unsupported dtype";
        case BD_E_PARAM: return "invalid parameter (mode, S, tau, scale or alignment)";
        case BD_E_WORKSPACE: return "workspace missing, misaligned or too small";
        case BD_E_LAUNCH: return "the HIP runtime rejected a kernel launch";
        case BD_E_SCRATCH: return "the call needs more than the fixed device scratch of bd_attn_step_noalloc";
        default: return "unknown status";
    }
}

int32_t bd_last_hip_error(void) { return g_last_hip_error; }

}  // extern "C"

extern "C" {

size_t bd_two_stream_workspace_bytes(const bd_two_stream_desc *desc) {
    if (check_two_stream_desc(desc) != BD_OK) return SIZE_MAX;
    const bd::AttnPlan pl = bd::plan_attention(desc->n_seq, desc->Lc + desc->Ln, desc->Hq, desc->Hkv, desc->d,
                                               BD_BF16, 0, true);
    return pl.ws_bytes;
}

bd_status bd_two_stream_attn(const bd_two_stream_desc *desc, const void *q, const void *k, const void *v,
                             const int32_t *spans, const int32_t *n_spans, void *out, void *workspace,
                             size_t workspace_bytes, void *stream) {
    bd_status st = check_two_stream_desc(desc);
    if (st != BD_OK) return st;
    if (!q || !k || !v || !out) return BD_E_NULL;
    if (desc->max_spans > 0 && (!spans || !n_spans)) return BD_E_NULL;
    if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(out)) return BD_E_PARAM;
    const bd::AttnPlan pl = bd::plan_attention(desc->n_seq, desc->Lc + desc->Ln, desc->Hq, desc->Hkv, desc->d,
                                               BD_BF16, 0, true);
    if (pl.ws_bytes > 0 && (!workspace || workspace_bytes < pl.ws_bytes || !aligned16(workspace)))
        return BD_E_WORKSPACE;
    bd::AttnArgs a{};
    a.q = q;
    a.k_cache = k;
    a.v_cache = v;
    a.out = out;
    a.ws = workspace;
    a.n = desc->n_seq;
    a.D = desc->Lc + desc->Ln;
    a.Hq = desc->Hq;
    a.Hkv = desc->Hkv;
    a.d = desc->d;
    a.cap = desc->cap;
    a.scale = desc->scale;
    a.spans = spans;
    a.n_spans = n_spans;
    a.Lc = desc->Lc;
    a.max_spans = desc->max_spans;
    a.Dblk = desc->D;
    return launched(bd::launch_attention_mfma(pl, a, (hipStream_t)stream));
}

}  // extern "C"
