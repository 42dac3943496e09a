// Internal launch interface between the C-ABI layer (bd_api.hip) and the kernels.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace bd {

// ---- block attention -------------------------------------------------------
constexpr int kTileKeys = 32;       // keys per LDS tile (bf16; E4M3 tiles hold twice as many)
constexpr int kCUs = 256;           // compute units of an MI355X
constexpr int kNarrowSplits = 16;   // split-K pieces per unit in general
constexpr int kWideSplits = 32;     // ... and when every workgroup has a CU of its own
constexpr int kMaxSplits = 64;      // ... and when even 64 per unit leave that so

struct AttnPlan {
    bool mfma;            // MFMA path: bf16, or bf16 queries with E4M3 K/V (else the fp32 vector path)
    bool fp8;             // E4M3 K/V (64-key tiles)
    bool seq;             // two-stream mode: whole sequences, per-row key ranges
    int tk;               // keys per tile
    int nw;               // waves per workgroup (MFMA path)
    int rows;             // grouped query rows per (item, KV head) = D * Hq/Hkv
    int rows_per_group;   // rows one workgroup covers (32 * nw)
    int row_blocks;
    int units;            // n_items * Hkv * row_blocks
    int tiles_per_split;
    int max_splits;
    bool balanced;        // ragged-batch plan: split counts from the device-side prefix lengths
    int balance_slots;    // ... workgroups it may use
    bool pair;            // one 8-wave workgroup runs two list slots (two 4-wave halves)
    int max_prefix;       // the host's longest prefix
    int grid;             // workgroups launched
    size_t ws_ml_off, ws_o_off, ws_splits_off, ws_bytes;
};

struct AttnArgs {
    const void *q, *k_blk, *v_blk, *k_cache, *v_cache;
    const int32_t *prefix;
    const float *k_scale, *v_scale;  // E4M3 K/V only
    void *out;
    void *ws;
    int n, D, Hq, Hkv, d, cap, mode;
    int B;  // quadratic mode: draft block size (D is then the slot count B (B + 3) / 2)
    float scale;
    // two-stream mode (D = Lc + Ln positions per sequence)
    const int32_t *spans, *n_spans;
    int Lc, max_spans, Dblk;
};

constexpr int kBalancedMaxItems = 64;  // the balanced plan keeps one lane per item
AttnPlan plan_attention(int n, int D, int Hq, int Hkv, int d, int dtype, int max_prefix, bool seq = false,
                        bool balanced = false);
hipError_t launch_attention_mfma(const AttnPlan &plan, const AttnArgs &a, hipStream_t s);
hipError_t launch_attention_vec(const AttnArgs &a, int dtype, hipStream_t s);

// ---- confidence / verify ----------------------------------------------------
struct RowPlan {
    int groups;    // workgroups per request
    int max_cpr;   // most chunks one participating row is cut into
    size_t part_off, grp_off, cnt_off, ws_bytes;
    bool ok;       // the grid fits one launch
};
RowPlan plan_rows(int n_req, int D, int V);

struct RowArgs {
    const float *logits;
    uint8_t *masked;
    int32_t *tokens;
    float *conf;
    int32_t *argmax;
    uint8_t *committed;
    int32_t *n_committed;
    const int32_t *draft;
    int32_t *accepted_len;
    void *ws;
    int n_req, D, V, S;
    float tau;
};
hipError_t launch_confidence_commit(const RowPlan &plan, const RowArgs &a, hipStream_t s);
hipError_t launch_spec_verify(const RowPlan &plan, const RowArgs &a, hipStream_t s);

// ---- LM head + confidence + commit ------------------------------------------
struct LhPlan {
    int R;               // block slots = n_req * D (<= 16)
    int tiles;           // 16-row vocabulary tiles
    int tiles_per_wave;
    int G;               // workgroups
    size_t lds;          // dynamic LDS: the hidden states, 16 rows of H + 8
    size_t ms_off, i_off, grp_off, cnt_off, ws_bytes;
    bool ok;             // G within the finisher's reach
};
LhPlan plan_lmhead(int n_req, int D, int V, int H);

struct LhArgs {
    const void *hidden, *weight;
    uint8_t *masked;
    int32_t *tokens;
    float *conf;
    int32_t *argmax;
    uint8_t *committed;
    int32_t *n_committed;
    void *ws;
    int n_req, D, V, H, S;
    float tau;
};
hipError_t launch_lmhead(const LhPlan &plan, const LhArgs &a, hipStream_t s);

// ---- KV append --------------------------------------------------------------
// D: most slots an item may append; S: block slots per item (the row stride of k_blk / v_blk).
hipError_t launch_kv_append(int n, int D, int S, int Hkv, int d, int cap, int elem_bytes, void *k_cache,
                            void *v_cache, int32_t *prefix, const void *k_blk, const void *v_blk,
                            const int32_t *n_accept, int32_t *dev_err, hipStream_t s);

}  // namespace bd
