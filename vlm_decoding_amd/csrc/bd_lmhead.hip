// Vocabulary projection (LM head) of one denoising step fused with its
// confidence + commit, on gfx950.
//
// The step's logits are the final hidden state of every block slot times the
// vocabulary projection, logits[r][v] = sum_h hidden[r][h] * weight[v][h];
// their softmax gives each masked slot's greedy token and confidence, which
// the commit rule reads (DiffusionVL notes, cached block decoding and
// Algorithm 1).  Here the logits never leave registers: the kernel streams the
// weight matrix (the step's dominant bytes: V x H bf16) once, and each lane
// folds the logits it forms into a running (max, first argmax, sum of
// exp(x - max)) per slot.
//
// Layout of the work.  The R <= 16 slots are the N dimension of
// v_mfma_f32_16x16x32_bf16; vocabulary rows are its M dimension.  Every wave
// owns a contiguous range of 16-row vocabulary tiles and runs through them
// with the weight loads three 256-column blocks ahead (register ring), so its
// loads never wait on its MFMAs.  Load j of a step covers columns 32j..32j+31
// of the block for all 16 rows (each row's 64 bytes contiguous; a step reads
// 512 contiguous bytes of every row, which measured faster than narrower
// steps); the hidden states sit in LDS (rows padded by 16 bytes, so the 16
// rows of one MFMA operand fall in distinct banks).  The
// workgroup's per-slot partials go out with write-through stores; the last
// workgroup (two levels of tickets) merges them in workgroup order and commits.  No float
// atomics: results are identical run to run.
#include "bd_common.h"
#include "bd_internal.h"
#include "bd_rowreduce.h"

namespace bd {
namespace {

constexpr int LH_NT = 256;      // four waves
constexpr int LH_SLOTS = 16;    // MFMA N dimension (slots, zero-padded)
constexpr int LH_BLK = 256;     // hidden columns per pipeline step (eight MFMAs)
constexpr int LH_RING = 4;      // register ring: loads run LH_RING - 1 steps ahead
constexpr int LH_LPS = LH_BLK / 32;  // 16-byte loads (and MFMAs) per lane and step
// Tickets on one address are served one after another (about 10 ns each), so
// workgroups ticket a counter per group of kLhTicketGroup and the last of a
// group tickets the call; each counter has a 256-byte line of its own.
constexpr int kLhTicketGroup = 16;
constexpr int kLhCounterStride = 64;

struct LhParams {
    const uint16_t *hidden, *weight;
    uint8_t *masked;
    int32_t *tokens;
    float *conf;
    int32_t *argmax;
    uint8_t *committed;
    int32_t *n_committed;
    float2 *part_ms;  // [G][16] (max, sum)
    int *part_i;      // [G][16] first argmax
    int *grp_cnt;     // [NG] first-level tickets, kLhCounterStride ints apart
    int *cnt;         // second-level ticket
    int n_req, D, R, V, H, S, tiles, tiles_per_wave, G, NG;
    float tau;
};

__global__ __launch_bounds__(LH_NT, 2) void lmhead_kernel(LhParams p) {
    extern __shared__ __attribute__((aligned(16))) uint16_t xs[];  // [16][H + 8]
    __shared__ Part s_part[LH_NT / 64][LH_SLOTS];
    __shared__ __attribute__((aligned(16))) float s_conf[64];
    __shared__ int s_arg[64];
    __shared__ int s_done;
    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int w = tid >> 6;
    const int XS = p.H + 8;
    const int NHB = p.H / LH_BLK;

    // Hidden states of the R slots (zero rows up to 16), 16 bytes per thread.
    {
        const int upr = p.H / 8;
        for (int u = tid; u < LH_SLOTS * upr; u += LH_NT) {
            const int row = u / upr, c = u - row * upr;
            uint4 v = make_uint4(0u, 0u, 0u, 0u);
            if (row < p.R) v = *reinterpret_cast<const uint4 *>(p.hidden + (size_t)row * p.H + c * 8);
            *reinterpret_cast<uint4 *>(&xs[row * XS + c * 8]) = v;
        }
    }
    __syncthreads();

    // This wave's tiles and pipeline steps (tile-major, LH_BLK hidden columns a step).
    const int gw = blockIdx.x * (LH_NT / 64) + w;
    const int t_beg = min(p.tiles, gw * p.tiles_per_wave);
    const int t_end = min(p.tiles, t_beg + p.tiles_per_wave);
    const int nsteps = (t_end - t_beg) * NHB;
    const int n = lane & 15;    // slot column of the MFMA operands and results
    const int kq = lane >> 4;   // which 8 columns of each 32-column MFMA chunk
    const uint16_t *xrow = xs + n * XS + 8 * kq;

    // Every step has the same shape - issue the loads of step q + 3, then two
    // MFMAs on the block loaded three steps earlier - so the compiler can wait
    // for exactly the loads it needs.  The step count is rounded up to the
    // ring size; loads past the wave's last step read one fixed, cached row.
    uint4 ring[LH_RING][LH_LPS];
    int lt = t_beg, lb = 0;  // load cursor: tile, column block
    auto load = [&](uint4 (&dst)[LH_LPS], bool real) __attribute__((always_inline)) {
        const int vrow = min(lt * 16 + n, p.V - 1);  // rows past V are formed but never used
        const uint16_t *src = real ? p.weight + (size_t)vrow * p.H + lb * LH_BLK + 8 * kq : p.weight;
#pragma unroll
        for (int j = 0; j < LH_LPS; ++j) dst[j] = *reinterpret_cast<const uint4 *>(src + 32 * j);
        if (++lb == NHB) {
            lb = 0;
            ++lt;
        }
    };
#pragma unroll
    for (int j = 0; j < LH_RING - 1; ++j) load(ring[j], j < nsteps);

    Part run{-INFINITY, 0.f, 0x7fffffff};
    floatx4 acc = {0.f, 0.f, 0.f, 0.f};
    int ct = t_beg, cb = 0;  // compute cursor
    auto step = [&](auto slot, int q) __attribute__((always_inline)) {
        constexpr int J = decltype(slot)::value;
        load(ring[(J + LH_RING - 1) % LH_RING], q + LH_RING - 1 < nsteps);
        if (q < nsteps) {
            // MFMA j: lane (n, kq) supplies weight row n and slot n's hidden state at
            // the same eight columns, 32j + 8kq .. +7 of the block.
#pragma unroll
            for (int j = 0; j < LH_LPS; ++j) {
                const bf16x8 xj = *reinterpret_cast<const bf16x8 *>(xrow + cb * LH_BLK + 32 * j);
                acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(*reinterpret_cast<const bf16x8 *>(&ring[J][j]), xj, acc,
                                                              0, 0, 0);
            }
            if (++cb == NHB) {
                // Tile done: this lane holds vocabulary rows 16*ct + 4*kq + i of slot n.
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    const int v = ct * 16 + 4 * kq + i;
                    if (v < p.V) push<true>(run, acc[i], v);
                }
                acc = floatx4{0.f, 0.f, 0.f, 0.f};
                cb = 0;
                ++ct;
            }
        }
    };
    const int nsteps_r = (nsteps + LH_RING - 1) / LH_RING * LH_RING;
    for (int q = 0; q < nsteps_r; q += LH_RING) {
        step(std::integral_constant<int, 0>{}, q);
        step(std::integral_constant<int, 1>{}, q + 1);
        step(std::integral_constant<int, 2>{}, q + 2);
        step(std::integral_constant<int, 3>{}, q + 3);
    }

    // Slot n's partial over this wave's vocabulary: lanes n, n+16, n+32, n+48.
    run = swap_part<true>(swap_part<false>(run));
    if (lane < LH_SLOTS) s_part[w][lane] = run;
    __syncthreads();
    if (tid < LH_SLOTS) {
        Part t = s_part[0][tid];
#pragma unroll
        for (int k = 1; k < LH_NT / 64; ++k) t = combine(t, s_part[k][tid]);
        const size_t o = (size_t)blockIdx.x * LH_SLOTS + tid;
        bd_coherent_store2(reinterpret_cast<float *>(&p.part_ms[o]), t.m, t.s);
        bd_coherent_store(p.part_i + o, t.i);
    }
    bd_wait_all_memory();
    __syncthreads();
    if (tid == 0) {
        const int grp = blockIdx.x / kLhTicketGroup;
        const int gsize = min(kLhTicketGroup, p.G - grp * kLhTicketGroup);
        int *gc = p.grp_cnt + (size_t)grp * kLhCounterStride;
        bool last = false;
        if (bd_ticket(gc) == gsize - 1) {
            bd_coherent_store(gc, 0);  // every ticket of the group is taken: reset for the next call
            last = p.NG == 1 || bd_ticket(p.cnt) == p.NG - 1;
        }
        s_done = last;
    }
    __syncthreads();
    if (!s_done) return;

    // Last workgroup: sixteen lanes per slot merge the G workgroup partials
    // (lane c takes workgroups c, c + 16, ... in order, all loads issued
    // before use), then a fixed 16-lane tree.
    {
        constexpr int MAXC = 512 / 16;  // G <= 512
        const int slot = tid >> 4, c0 = tid & 15;
        float2 ms[MAXC];
        int ix[MAXC];
#pragma unroll
        for (int j = 0; j < MAXC; ++j) {
            const int c = c0 + 16 * j;
            if (c < p.G && slot < p.R) {
                const size_t o = (size_t)c * LH_SLOTS + slot;
                ms[j] = bd_coherent_load2(reinterpret_cast<const float *>(&p.part_ms[o]));
                ix[j] = bd_coherent_load(p.part_i + o);
            }
        }
        Part t{-INFINITY, 0.f, 0x7fffffff};
#pragma unroll
        for (int j = 0; j < MAXC; ++j)
            if (c0 + 16 * j < p.G && slot < p.R) t = combine(t, Part{ms[j].x, ms[j].y, ix[j]});
        t = reduce16(t);
        if (c0 == 0 && slot < p.R) {
            s_conf[slot] = 1.0f / t.s;
            s_arg[slot] = t.i;
        }
    }
    __syncthreads();
    // One wave commits each request in turn (slots r*D .. r*D + D - 1).
    if (w == 0) {
        for (int r = 0; r < p.n_req; ++r) {
            const size_t ob = (size_t)r * p.D;
            const bool mk = lane < p.D && p.masked[ob + lane] != 0;
            const unsigned long long mask = __builtin_amdgcn_ballot_w64(mk);
            const unsigned long long tb =
                commit_request(s_conf + r * p.D, s_arg + r * p.D, mask, __popcll(mask), p.D, p.S, p.tau, lane,
                               p.masked + ob, p.tokens + ob, p.conf ? p.conf + ob : nullptr,
                               p.argmax ? p.argmax + ob : nullptr, p.committed ? p.committed + ob : nullptr);
            if (lane == 0 && p.n_committed) p.n_committed[r] = __popcll(tb);
        }
        if (lane == 0) bd_coherent_store(p.cnt, 0);
    }
}

}  // namespace

LhPlan plan_lmhead(int n_req, int D, int V, int H) {
    LhPlan pl{};
    pl.R = n_req * D;
    pl.tiles = (V + 15) / 16;
    pl.lds = (size_t)LH_SLOTS * (H + 8) * 2;
    // Workgroups resident at once: two per CU while the hidden states fit
    // twice in the 160 KB of LDS, else one.
    const int per_cu = 2 * (pl.lds + 2048) <= 160 * 1024 ? 2 : 1;  // + the static LDS
    const int waves_max = kCUs * per_cu * (LH_NT / 64);
    pl.tiles_per_wave = (pl.tiles + waves_max - 1) / waves_max;
    const int waves = (pl.tiles + pl.tiles_per_wave - 1) / pl.tiles_per_wave;
    pl.G = (waves + (LH_NT / 64) - 1) / (LH_NT / 64);
    size_t off = 0;
    auto take = [&](size_t bytes) {
        size_t o = off;
        off += (bytes + 255) / 256 * 256;
        return o;
    };
    pl.ms_off = take(sizeof(float) * 2 * LH_SLOTS * (size_t)pl.G);
    pl.i_off = take(sizeof(int) * LH_SLOTS * (size_t)pl.G);
    pl.grp_off = take(sizeof(int) * kLhCounterStride * (size_t)((pl.G + kLhTicketGroup - 1) / kLhTicketGroup));
    pl.cnt_off = take(sizeof(int));
    pl.ws_bytes = off;
    pl.ok = pl.G <= 512;
    return pl;
}

hipError_t launch_lmhead(const LhPlan &pl, const LhArgs &a, hipStream_t s) {
    LhParams p{};
    p.hidden = (const uint16_t *)a.hidden;
    p.weight = (const uint16_t *)a.weight;
    p.masked = a.masked;
    p.tokens = a.tokens;
    p.conf = a.conf;
    p.argmax = a.argmax;
    p.committed = a.committed;
    p.n_committed = a.n_committed;
    char *ws = (char *)a.ws;
    p.part_ms = (float2 *)(ws + pl.ms_off);
    p.part_i = (int *)(ws + pl.i_off);
    p.grp_cnt = (int *)(ws + pl.grp_off);
    p.cnt = (int *)(ws + pl.cnt_off);
    p.n_req = a.n_req;
    p.D = a.D;
    p.R = pl.R;
    p.V = a.V;
    p.H = a.H;
    p.S = a.S;
    p.tiles = pl.tiles;
    p.tiles_per_wave = pl.tiles_per_wave;
    p.G = pl.G;
    p.NG = (pl.G + kLhTicketGroup - 1) / kLhTicketGroup;
    p.tau = a.tau;
    if (pl.lds > 64 * 1024) {
        const hipError_t e = hipFuncSetAttribute((const void *)lmhead_kernel,
                                                 hipFuncAttributeMaxDynamicSharedMemorySize, (int)pl.lds);
        if (e != hipSuccess) return e;
    }
    hipLaunchKernelGGL(lmhead_kernel, dim3(pl.G), dim3(LH_NT), pl.lds, s, p);
    return hipGetLastError();
}

}  // namespace bd
