// Host side of the C ABI declared in include/moe.h: argument checks, the
// workspace layout, and the launch sequence of one forward.
#include <hip/hip_runtime.h>
#include <stdarg.h>
#include <stdio.h>
#include <string.h>

#include <mutex>
#include <string>

#include "../../include/moe.h"
#include "common.h"

namespace moe {
hipError_t launch_route(const float* logits, int64_t T_cap, const int32_t* live, int E, int k,
                        int32_t* ids, float* probs, WsHeader* hdr, int num_cu, hipStream_t s);
hipError_t launch_prep(const int32_t* ids, const float* probs, int64_t T_cap, const int32_t* live,
                       int E, int k, int num_cu, char* ws, const WsLayout& L, hipStream_t s,
                       int fin_H, int fin_mode, void* fin_out);
hipError_t launch_finalize(const float* O, const int32_t* dst, const float* sorted_probs,
                           int64_t T_cap, const int32_t* live, int k, int H, int mode, void* out,
                           int num_cu, hipStream_t s);
hipError_t launch_pack_bf16(const uint16_t* w1, const uint16_t* w2, uint8_t* kbuf, int E, int H,
                            int F, int num_cu, hipStream_t s);
hipError_t launch_pack_mxfp8(const uint16_t* w1, const uint16_t* w2, uint8_t* kbuf, int E, int H,
                             int F, int num_cu, hipStream_t s);
void mx_section_bytes(int E, int H, int F, size_t* c1, size_t* c2, size_t* s1, size_t* s2);
hipError_t launch_pack_mxfp4(const uint16_t* w1, const uint16_t* w2, uint8_t* kbuf, int E, int H,
                             int F, int num_cu, hipStream_t s);
void mx4_section_bytes(int E, int H, int F, size_t* c1, size_t* c2, size_t* s1, size_t* s2);
hipError_t launch_quant_x(const uint16_t* x, int64_t T_cap, const int32_t* live, int H,
                          uint8_t* codes, uint8_t* scales, int num_cu, hipStream_t s);
}  // namespace moe

#include "gemm_args.h"

namespace moe {
hipError_t launch_gemm_bf16(bool fc1, const GemmArgs& g, int num_cu, hipStream_t s, hipEvent_t t0,
                            hipEvent_t t1, hipStream_t s_small = nullptr);
hipError_t launch_gemm_bf16_fused(const GemmArgs& g1, const GemmArgs& g2, int num_cu, hipStream_t s,
                                  hipEvent_t t0, hipEvent_t t1);
hipError_t launch_gemm_mxfp8(bool fc1, bool w4, const MxGemmArgs& g, int num_cu, hipStream_t s,
                             hipEvent_t t0, hipEvent_t t1);
}  // namespace moe

using namespace moe;

struct moe_ctx {
    int E, H, F, k, precision;
    const uint8_t* kbuf = nullptr;   // not owned
    int num_cu = 0;
    int device = -1;
    hipEvent_t stage_events[6] = {};
    bool record_stages = false;
};

static hipError_t mark(moe_ctx* h, int i, hipStream_t s)
{
    return (h->record_stages && h->stage_events[i]) ? hipEventRecord(h->stage_events[i], s)
                                                     : hipSuccess;
}

// Stage event i if stage events are on (else null).  Events 2 and 3 bracket
// the FC1 + SwiGLU launch: they are handed to the launch itself, which records
// its own start and end (a separate event record before and after it would
// put marker packets in the stream, each costing ~5 us of idle GPU).
static hipEvent_t stage_event(const moe_ctx* h, int i)
{
    return h->record_stages ? h->stage_events[i] : nullptr;
}

static thread_local std::string g_err;

static moe_status fail(moe_status st, const char* fmt, ...)
    __attribute__((format(printf, 2, 3)));

static moe_status fail(moe_status st, const char* fmt, ...)
{
    char buf[512];
    va_list ap;
    va_start(ap, fmt);
    vsnprintf(buf, sizeof(buf), fmt, ap);
    va_end(ap);
    g_err = buf;
    return st;
}

static moe_status hip_fail(hipError_t e, const char* what)
{
    return fail(MOE_ERR_HIP, "%s: %s", what, hipGetErrorString(e));
}

static bool aligned16(const void* p) { return ((uintptr_t)p & 15u) == 0; }

static size_t up256(size_t v) { return (v + 255) / 256 * 256; }

static WsLayout layout_of(const moe_ctx* h, int64_t T_cap)
{
    WsLayout L;
    const int64_t E = h->E, H = h->H, F = h->F, k = h->k;
    const int64_t R = T_cap * k;
    L.nchunks = (T_cap + kChunkTok - 1) / kChunkTok;
    if (L.nchunks < 1) L.nchunks = 1;
    L.max_tiles = E + (R + kBM - 1) / kBM + 1;
    L.max_tiles_big = E + (R + kBigBMRows - 1) / kBigBMRows + 1;
    size_t o = 0;
    auto take = [&](size_t bytes) { size_t at = o; o += up256(bytes > 0 ? bytes : 1); return at; };
    L.hdr = take(sizeof(WsHeader));
    L.counts = take(4 * E);
    L.offsets = take(4 * (E + 1));
    L.chunk_base = take(4 * E * L.nchunks);
    L.chunk_err = take(4 * L.nchunks);
    L.local_rank = take(4 * R);
    L.sorted_ids = take(4 * R);
    L.sorted_probs = take(4 * R);
    L.perm_src = take(4 * R);
    L.dst = take(4 * R);
    L.tiles = take(8 * L.max_tiles);
    L.tiles_big = take(8 * L.max_tiles_big);
    L.ready = take(4 * (L.max_tiles + 4 * L.max_tiles_big));
    L.fin_cnt = take(4 * T_cap * ((H + kFinCols - 1) / kFinCols));
    if (h->precision == MOE_BF16) {
        L.hbuf = take(2 * R * F);
        L.hscale = 0;
        L.xq = L.xs = 0;
    } else {
        L.hbuf = take(R * F);
        L.hscale = take(R * (F / 32));
        L.xq = take(T_cap * H);
        L.xs = take(T_cap * (H / 32));
    }
    L.obuf = take(4 * R * H);
    L.total = o;
    return L;
}

static moe_status ensure_device(moe_ctx* h)
{
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return hip_fail(e, "hipGetDevice");
    if (h->device != dev || h->num_cu <= 0) {
        int cus = 0;
        e = hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev);
        if (e != hipSuccess) return hip_fail(e, "hipDeviceGetAttribute");
        h->device = dev;
        h->num_cu = cus > 0 ? cus : 1;
    }
    return MOE_OK;
}

// Workspace of moe_forward_noalloc: device memory the library itself holds, one
// copy per GPU (the array is a device global of this code object), kept until
// the process ends.  Host code never uses the array's name as an address: the
// name is a host-side stand-in, so the device address of each GPU's copy is
// taken once with hipGetSymbolAddress while that GPU is current.
constexpr size_t kScratchBytes = (size_t)64 << 20;
constexpr int kMaxScratchDevices = 64;
static __device__ __attribute__((aligned(256))) char scratch[kScratchBytes];
static void* g_scratch_ptr[kMaxScratchDevices];
static std::mutex g_scratch_mu;

static moe_status scratch_of_current_device(void** out)
{
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return hip_fail(e, "hipGetDevice");
    if (dev < 0 || dev >= kMaxScratchDevices)
        return fail(MOE_ERR_UNSUPPORTED, "device %d: at most %d devices", dev, kMaxScratchDevices);
    std::lock_guard<std::mutex> lock(g_scratch_mu);
    if (!g_scratch_ptr[dev]) {
        void* p = nullptr;
        e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
        if (e != hipSuccess) return hip_fail(e, "hipGetSymbolAddress(scratch)");
        if (!p) return fail(MOE_ERR_HIP, "hipGetSymbolAddress(scratch) returned NULL");
        g_scratch_ptr[dev] = p;
    }
    *out = g_scratch_ptr[dev];
    return MOE_OK;
}

// Side stream of the bf16 forward above a 1024-token capacity, where a GEMM
// stage is a 256-row launch and a 64-row launch over disjoint experts: the
// 64-row FC1 -> FC2 chain runs on the side stream while the 256-row chain runs
// on the caller's, so the 64-row tiles fill the CUs the 256-row launch frees at
// its tail.  One non-blocking stream (default priority) and a fork and a join
// event per GPU, created by moe_load_weights (a set-up call, outside any graph
// capture) and kept until the process ends.  g_side_mu serializes the
// record / wait pairs of concurrent forwards, so each fork and join pairs with
// its own forward's launches.
struct SideStream {
    hipStream_t s = nullptr;
    hipEvent_t fork = nullptr, join = nullptr;
};
static SideStream g_side[kMaxScratchDevices];
static std::mutex g_side_mu;

static moe_status ensure_side_stream(int dev)
{
    if (dev < 0 || dev >= kMaxScratchDevices) return MOE_OK;   // forwards there stay on one stream
    std::lock_guard<std::mutex> lock(g_side_mu);
    SideStream& ss = g_side[dev];
    if (ss.s) return MOE_OK;
    hipError_t e = hipStreamCreateWithFlags(&ss.s, hipStreamNonBlocking);
    if (e == hipSuccess) e = hipEventCreateWithFlags(&ss.fork, hipEventDisableTiming);
    if (e == hipSuccess) e = hipEventCreateWithFlags(&ss.join, hipEventDisableTiming);
    if (e != hipSuccess) {
        if (ss.join) (void)hipEventDestroy(ss.join);
        if (ss.fork) (void)hipEventDestroy(ss.fork);
        if (ss.s) (void)hipStreamDestroy(ss.s);
        ss = SideStream();
        return hip_fail(e, "moe_load_weights: side stream");
    }
    return MOE_OK;
}

extern "C" {

const char* moe_last_error(void) { return g_err.c_str(); }

moe_status moe_create(int E, int H, int F, int topk, int precision, moe_handle* out)
{
    if (!out) return fail(MOE_ERR_INVALID_ARG, "moe_create: out is NULL");
    *out = nullptr;
    if (precision != MOE_BF16 && precision != MOE_MXFP8 && precision != MOE_MXFP4)
        return fail(MOE_ERR_UNSUPPORTED,
                    "moe_create: precision %d is not supported (bf16=0, mxfp8=1, mxfp4=2)", precision);
    if (E < 1 || E > kMaxExperts)
        return fail(MOE_ERR_INVALID_ARG, "moe_create: E=%d outside [1, %d]", E, kMaxExperts);
    if (topk < 1 || topk > kMaxTopk || topk > E)
        return fail(MOE_ERR_INVALID_ARG, "moe_create: topk=%d outside [1, min(E, %d)]", topk, kMaxTopk);
    if (H <= 0 || H % 32 != 0)
        return fail(MOE_ERR_INVALID_ARG, "moe_create: H=%d must be a positive multiple of 32", H);
    if (F <= 0 || F % 32 != 0)
        return fail(MOE_ERR_INVALID_ARG, "moe_create: F=%d must be a positive multiple of 32", F);
    moe_ctx* h = new moe_ctx();
    h->E = E; h->H = H; h->F = F; h->k = topk; h->precision = precision;
    *out = h;
    g_err.clear();
    return MOE_OK;
}

void moe_destroy(moe_handle h) { delete h; }

size_t moe_weight_bytes(moe_handle h)
{
    if (!h) return 0;
    size_t n1 = (size_t)h->E * 2 * h->F * h->H, n2 = (size_t)h->E * h->H * h->F;
    if (h->precision == MOE_BF16) return 2 * (n1 + n2);
    size_t c1, c2, s1, s2;
    if (h->precision == MOE_MXFP4)
        mx4_section_bytes(h->E, h->H, h->F, &c1, &c2, &s1, &s2);
    else
        mx_section_bytes(h->E, h->H, h->F, &c1, &c2, &s1, &s2);
    return c1 + c2 + s1 + s2;
}

size_t moe_workspace_bytes(moe_handle h, int64_t T_cap)
{
    if (!h || T_cap < 0) return 0;
    return layout_of(h, T_cap).total;
}

moe_status moe_load_weights(moe_handle h, const void* w1, const void* w2, void* kbuf,
                            size_t kbuf_bytes, hipStream_t stream)
{
    if (!h) return fail(MOE_ERR_INVALID_ARG, "moe_load_weights: NULL handle");
    if (!w1 || !w2 || !kbuf) return fail(MOE_ERR_INVALID_ARG, "moe_load_weights: NULL pointer");
    if (!aligned16(w1) || !aligned16(w2) || !aligned16(kbuf))
        return fail(MOE_ERR_INVALID_ARG, "moe_load_weights: pointers must be 16-byte aligned");
    if (kbuf_bytes < moe_weight_bytes(h))
        return fail(MOE_ERR_INVALID_ARG, "moe_load_weights: kbuf_bytes %zu < %zu", kbuf_bytes,
                    moe_weight_bytes(h));
    moe_status st = ensure_device(h);
    if (st != MOE_OK) return st;
    if (h->precision == MOE_BF16 && (st = ensure_side_stream(h->device)) != MOE_OK) return st;
    const uint16_t* a = (const uint16_t*)w1;
    const uint16_t* b = (const uint16_t*)w2;
    uint8_t* kb = (uint8_t*)kbuf;
    hipError_t e =
        h->precision == MOE_BF16    ? launch_pack_bf16(a, b, kb, h->E, h->H, h->F, h->num_cu, stream)
        : h->precision == MOE_MXFP8 ? launch_pack_mxfp8(a, b, kb, h->E, h->H, h->F, h->num_cu, stream)
                                    : launch_pack_mxfp4(a, b, kb, h->E, h->H, h->F, h->num_cu, stream);
    if (e != hipSuccess) return hip_fail(e, "moe_load_weights: launch");
    h->kbuf = (const uint8_t*)kbuf;
    return MOE_OK;
}

moe_status moe_route(moe_handle h, const float* logits, int64_t T_cap,
                     const int32_t* live_rows_dev, int32_t* ids, float* probs, void* ws,
                     size_t ws_bytes, hipStream_t stream)
{
    if (!h) return fail(MOE_ERR_INVALID_ARG, "moe_route: NULL handle");
    if (T_cap < 0 || T_cap > (int64_t)1 << 26)
        return fail(MOE_ERR_INVALID_ARG, "moe_route: T_cap=%lld out of range", (long long)T_cap);
    if (!logits || !live_rows_dev || !ids || !probs || !ws)
        return fail(MOE_ERR_INVALID_ARG, "moe_route: NULL pointer");
    if (ws_bytes < sizeof(WsHeader))
        return fail(MOE_ERR_INVALID_ARG, "moe_route: workspace too small");
    if (!aligned16(logits) || !aligned16(ids) || !aligned16(probs) || !aligned16(ws))
        return fail(MOE_ERR_INVALID_ARG, "moe_route: pointers must be 16-byte aligned");
    moe_status st = ensure_device(h);
    if (st != MOE_OK) return st;
    if (T_cap == 0) return MOE_OK;
    hipError_t e = launch_route(logits, T_cap, live_rows_dev, h->E, h->k, ids, probs,
                                (WsHeader*)ws, h->num_cu, stream);
    if (e != hipSuccess) return hip_fail(e, "moe_route: launch");
    return MOE_OK;
}

moe_status moe_forward(moe_handle h, const void* x, const int32_t* expert_ids,
                       const float* probs, int64_t T_cap, const int32_t* live_rows_dev,
                       float* out, void* ws, size_t ws_bytes, hipStream_t stream)
{
    return moe_forward_ex(h, x, expert_ids, probs, T_cap, live_rows_dev, MOE_COMBINE_FP32, out, ws,
                          ws_bytes, stream);
}

moe_status moe_forward_ex(moe_handle h, const void* x, const int32_t* expert_ids,
                          const float* probs, int64_t T_cap, const int32_t* live_rows_dev,
                          int combine, void* out, void* ws, size_t ws_bytes, hipStream_t stream)
{
    if (!h) return fail(MOE_ERR_INVALID_ARG, "moe_forward: NULL handle");
    if (!h->kbuf) return fail(MOE_ERR_NOT_LOADED, "moe_forward: no weights loaded (moe_load_weights)");
    if (T_cap < 0 || T_cap > (int64_t)1 << 26)
        return fail(MOE_ERR_INVALID_ARG, "moe_forward: T_cap=%lld out of range", (long long)T_cap);
    const bool fc1_topk = (combine & MOE_APPLY_TOPK_IN_FC1) != 0;
    // the single-launch finalize implies the single-launch FFN
    const bool fused_fin = (combine & MOE_FUSED_FINALIZE) != 0;
    const bool fused = fused_fin || (combine & MOE_FUSED_FFN) != 0;
    combine &= ~(MOE_APPLY_TOPK_IN_FC1 | MOE_FUSED_FFN | MOE_FUSED_FINALIZE);
    if (combine != MOE_COMBINE_FP32 && combine != MOE_COMBINE_BF16 && combine != MOE_COMBINE_ROWS)
        return fail(MOE_ERR_INVALID_ARG, "moe_forward: unknown combine %d", combine);
    if (fc1_topk && combine == MOE_COMBINE_ROWS)
        return fail(MOE_ERR_INVALID_ARG,
                    "moe_forward: MOE_APPLY_TOPK_IN_FC1 with row mode (which uses no probabilities)");
    if (fused && h->precision != MOE_BF16)
        return fail(MOE_ERR_INVALID_ARG, "moe_forward: %s is implemented for bf16 only",
                    fused_fin ? "MOE_FUSED_FINALIZE" : "MOE_FUSED_FFN");
    // row mode does not use the probabilities (every route has probability 1)
    if (!x || !expert_ids || (!probs && combine != MOE_COMBINE_ROWS) || !live_rows_dev || !out ||
        !ws)
        return fail(MOE_ERR_INVALID_ARG, "moe_forward: NULL pointer");
    if (!aligned16(x) || !aligned16(expert_ids) || (probs && !aligned16(probs)) ||
        !aligned16(out) || !aligned16(ws))
        return fail(MOE_ERR_INVALID_ARG, "moe_forward: pointers must be 16-byte aligned");
    const WsLayout L = layout_of(h, T_cap);
    if (ws_bytes < L.total)
        return fail(MOE_ERR_INVALID_ARG, "moe_forward: ws_bytes %zu < %zu for T_cap=%lld", ws_bytes,
                    L.total, (long long)T_cap);
    moe_status st = ensure_device(h);
    if (st != MOE_OK) return st;
    if (T_cap == 0) return MOE_OK;
    char* w = (char*)ws;
    WsHeader* hdr = (WsHeader*)(w + L.hdr);
    hipError_t e = mark(h, 0, stream);
    if (e != hipSuccess) return hip_fail(e, "moe_forward: stage event");
    e = launch_prep(expert_ids, probs, T_cap, live_rows_dev, h->E, h->k, h->num_cu, w, L, stream,
                    h->H, combine, fused_fin ? out : nullptr);
    if (e != hipSuccess) return hip_fail(e, "moe_forward: prep launch");
    if ((e = mark(h, 1, stream)) != hipSuccess) return hip_fail(e, "moe_forward: stage event");
    const int E = h->E, H = h->H, F = h->F;
    if (h->precision == MOE_BF16) {
        GemmArgs g1;
        g1.A = (const uint16_t*)x;
        g1.W = (const uint16_t*)h->kbuf;
        g1.perm_src = (const int32_t*)(w + L.perm_src);
        g1.tiles = (const int2*)(w + L.tiles);
        g1.tiles_big = (const int2*)(w + L.tiles_big);
        g1.offsets = (const int32_t*)(w + L.offsets);
        g1.hdr = hdr;
        g1.out = w + L.hbuf;
        g1.N = 2 * F;
        g1.K = H;
        g1.topk = h->k;
        g1.n_tiles_n = ((2 * F / 64) + 3) / 4;
        g1.max_tiles = (int)L.max_tiles;
        // the 256-row design: capacities above 1024, K a multiple of its 64-wide
        // stage, and byte offsets inside x and inside one expert's weights that
        // fit its 32-bit buffer offsets
        g1.small_takes_big = T_cap <= 1024 || H % 64 != 0 || H < 128 ||
                             (int64_t)T_cap * H * 2 >= ((int64_t)1 << 31) ||
                             (int64_t)2 * F * H * 2 >= ((int64_t)1 << 31);
        g1.row_prob = fc1_topk ? (const float*)(w + L.sorted_probs) : nullptr;
        g1.ready = (int32_t*)(w + L.ready);
        g1.err = &hdr->err;
        if (fused) g1.small_takes_big = 1;
        GemmArgs g2 = g1;
        g2.A = (const uint16_t*)(w + L.hbuf);
        g2.W = (const uint16_t*)h->kbuf + (size_t)E * 2 * F * H;
        g2.perm_src = nullptr;
        g2.out = w + L.obuf;
        g2.N = H;
        g2.K = F;
        g2.n_tiles_n = ((H + 63) / 64 + 3) / 4;
        g2.row_prob = nullptr;
        g2.small_takes_big = T_cap <= 1024 || F % 64 != 0 || F < 128 || (int64_t)H * F * 2 >= ((int64_t)1 << 31);
        g1.fin_cnt = g2.fin_cnt = nullptr;
        if (fused_fin) {
            // the FC2 tiles combine each token's 512-column blocks as they complete
            g2.fin_cnt = (int32_t*)(w + L.fin_cnt);
            g2.fin_route = (const int32_t*)(w + L.perm_src);
            g2.fin_dst = (const int32_t*)(w + L.dst);
            // with the probabilities applied inside FC1, or in row mode, every p is 1
            g2.fin_prob = (fc1_topk || combine == MOE_COMBINE_ROWS) ? nullptr
                                                                     : (const float*)(w + L.sorted_probs);
            g2.fin_out = out;
            g2.fin_mode = combine;
        }
        if (fused) {
            // one persistent launch, the 64-row design taking every tile; the
            // FC1 stage's events bracket it
            g2.small_takes_big = 1;
            e = launch_gemm_bf16_fused(g1, g2, h->num_cu, stream, stage_event(h, 2), stage_event(h, 3));
            if (e != hipSuccess) return hip_fail(e, "moe_forward: fused FFN launch");
        } else {
            const bool split1 = !g1.small_takes_big, split2 = !g2.small_takes_big;
            const SideStream* ss = (h->device >= 0 && h->device < kMaxScratchDevices)
                                       ? &g_side[h->device] : nullptr;
            // with stage events on (profiling) the stages stay serial, so that
            // the FC1 events bracket the whole stage.  The fork and join only
            // pay when the 64-row launches have tiles: forked while the
            // capacity's mean rows per expert, T_cap k / E, is under four
            // 128-row thresholds (bf16 at 4,096 tokens, 128 experts, top-8:
            // 748 -> 721-728 us/step); above it, as at 16,384 tokens, the
            // 64-row launches rarely find a tile and the stages stay serial
            const bool few_small = (int64_t)T_cap * h->k >= (int64_t)4 * kBigMin * E;
            if ((split1 || split2) && ss && ss->s && !h->record_stages && !few_small) {
                // the 256-row chain on `stream`, the 64-row chain on the side
                // stream: the two launches of a stage cover disjoint experts,
                // and FC2's tiles of a design read only the rows its own
                // design's FC1 tiles wrote; a stage of one launch (the 64-row
                // kernel taking every tile) waits for both chains
                std::lock_guard<std::mutex> lock(g_side_mu);
                auto fork = [&]() {
                    hipError_t r = hipEventRecord(ss->fork, stream);
                    return r == hipSuccess ? hipStreamWaitEvent(ss->s, ss->fork, 0) : r;
                };
                auto join = [&]() {
                    hipError_t r = hipEventRecord(ss->join, ss->s);
                    return r == hipSuccess ? hipStreamWaitEvent(stream, ss->join, 0) : r;
                };
                if (split1) {
                    if ((e = fork()) != hipSuccess) return hip_fail(e, "moe_forward: fork");
                    e = launch_gemm_bf16(true, g1, h->num_cu, stream, nullptr, nullptr, ss->s);
                    if (e != hipSuccess) return hip_fail(e, "moe_forward: FC1 launch");
                    if (!split2 && (e = join()) != hipSuccess) return hip_fail(e, "moe_forward: join");
                } else {
                    e = launch_gemm_bf16(true, g1, h->num_cu, stream, nullptr, nullptr);
                    if (e != hipSuccess) return hip_fail(e, "moe_forward: FC1 launch");
                    if (split2 && (e = fork()) != hipSuccess) return hip_fail(e, "moe_forward: fork");
                }
                e = launch_gemm_bf16(false, g2, h->num_cu, stream, nullptr, nullptr,
                                     split2 ? ss->s : nullptr);
                if (e != hipSuccess) return hip_fail(e, "moe_forward: FC2 launch");
                if (split2 && (e = join()) != hipSuccess) return hip_fail(e, "moe_forward: join");
            } else {
                e = launch_gemm_bf16(true, g1, h->num_cu, stream, stage_event(h, 2), stage_event(h, 3));
                if (e != hipSuccess) return hip_fail(e, "moe_forward: FC1 launch");
                e = launch_gemm_bf16(false, g2, h->num_cu, stream, nullptr, nullptr);
                if (e != hipSuccess) return hip_fail(e, "moe_forward: FC2 launch");
            }
        }
        if ((e = mark(h, 4, stream)) != hipSuccess) return hip_fail(e, "moe_forward: stage event");
    } else {
        // MXFP8, or MXFP4 weights with MXFP8 activations
        const bool w4 = h->precision == MOE_MXFP4;
        size_t b1, b2, b3, b4;
        if (w4)
            mx4_section_bytes(E, H, F, &b1, &b2, &b3, &b4);
        else
            mx_section_bytes(E, H, F, &b1, &b2, &b3, &b4);
        const uint8_t* c1 = h->kbuf;
        const uint8_t* c2 = c1 + b1;
        const uint8_t* s1 = c2 + b2;
        const uint8_t* s2 = s1 + b3;
        e = launch_quant_x((const uint16_t*)x, T_cap, live_rows_dev, H, (uint8_t*)(w + L.xq),
                           (uint8_t*)(w + L.xs), h->num_cu, stream);
        if (e != hipSuccess) return hip_fail(e, "moe_forward: quant-x launch");
        MxGemmArgs g1{};
        g1.A = (const uint8_t*)(w + L.xq);
        g1.As = (const uint8_t*)(w + L.xs);
        g1.W = c1;
        g1.Ws = s1;
        g1.perm_src = (const int32_t*)(w + L.perm_src);
        g1.tiles = (const int2*)(w + L.tiles);
        g1.tiles_big = (const int2*)(w + L.tiles_big);
        g1.offsets = (const int32_t*)(w + L.offsets);
        g1.hdr = hdr;
        g1.out = w + L.hbuf;
        g1.out_scale = (uint8_t*)(w + L.hscale);
        g1.N = 2 * F;
        g1.K = H;
        g1.topk = h->k;
        g1.n_tiles_n = ((2 * F / 64) + 3) / 4;
        // the 256-row LDS-staged tiles take K multiples of 128 and address their
        // operands with 32-bit buffer offsets (activation rows x K, one expert's
        // weight section); other shapes go to the streaming tiles
        g1.stream_big = H % 128 != 0 || T_cap * H >= ((int64_t)1 << 31) ||
                        (int64_t)2 * F * H >= ((int64_t)1 << 31);
        g1.small_batch = T_cap <= 1024;
        g1.a_bytes = T_cap * H;
        g1.row_prob = fc1_topk ? (const float*)(w + L.sorted_probs) : nullptr;
        e = launch_gemm_mxfp8(true, w4, g1, h->num_cu, stream, stage_event(h, 2), stage_event(h, 3));
        if (e != hipSuccess) return hip_fail(e, "moe_forward: FC1 launch");
        MxGemmArgs g2 = g1;
        g2.A = (const uint8_t*)(w + L.hbuf);
        g2.As = (const uint8_t*)(w + L.hscale);
        g2.W = c2;
        g2.Ws = s2;
        g2.perm_src = nullptr;
        g2.out = w + L.obuf;
        g2.out_scale = nullptr;
        g2.N = H;
        g2.K = F;
        g2.n_tiles_n = ((H + 63) / 64 + 3) / 4;
        g2.stream_big = F % 128 != 0 || (int64_t)H * F >= ((int64_t)1 << 31);
        g2.a_bytes = T_cap * h->k * F;
        g2.row_prob = nullptr;
        e = launch_gemm_mxfp8(false, w4, g2, h->num_cu, stream, nullptr, nullptr);
        if (e != hipSuccess) return hip_fail(e, "moe_forward: FC2 launch");
        if ((e = mark(h, 4, stream)) != hipSuccess) return hip_fail(e, "moe_forward: stage event");
    }
    if (fused_fin) {
        // the fused launch combined every live token
        if ((e = mark(h, 5, stream)) != hipSuccess) return hip_fail(e, "moe_forward: stage event");
        return MOE_OK;
    }
    // with the probabilities applied inside FC1 the finalize adds the rows
    e = launch_finalize((const float*)(w + L.obuf), (const int32_t*)(w + L.dst),
                        fc1_topk ? nullptr : (const float*)(w + L.sorted_probs), T_cap,
                        live_rows_dev, h->k, H, combine, out, h->num_cu, stream);
    if (e != hipSuccess) return hip_fail(e, "moe_forward: finalize launch");
    if ((e = mark(h, 5, stream)) != hipSuccess) return hip_fail(e, "moe_forward: stage event");
    return MOE_OK;
}

moe_status moe_forward_noalloc(moe_handle h, const void* x, const int32_t* expert_ids,
                               const float* probs, int64_t T_cap, const int32_t* live_rows_dev,
                               int combine, void* out, hipStream_t stream)
{
    if (!h) return fail(MOE_ERR_INVALID_ARG, "moe_forward_noalloc: NULL handle");
    if (T_cap < 0 || T_cap > (int64_t)1 << 26)
        return fail(MOE_ERR_INVALID_ARG, "moe_forward_noalloc: T_cap=%lld out of range",
                    (long long)T_cap);
    const size_t need = layout_of(h, T_cap).total;
    if (need > kScratchBytes)
        return fail(MOE_ERR_INVALID_ARG,
                    "moe_forward_noalloc: T_cap=%lld needs a %zu-byte workspace, above the "
                    "%zu-byte library scratch; use moe_forward with a caller workspace",
                    (long long)T_cap, need, kScratchBytes);
    void* ws = nullptr;
    moe_status st = scratch_of_current_device(&ws);
    if (st != MOE_OK) return st;
    return moe_forward_ex(h, x, expert_ids, probs, T_cap, live_rows_dev, combine, out, ws,
                          kScratchBytes, stream);
}

moe_status moe_get_indices(moe_handle h, const void* ws, int64_t T_cap, int32_t* counts,
                           int32_t* offsets, int32_t* perm_src, int32_t* dst,
                           int32_t* n_rows_out, int32_t* T_out, hipStream_t stream)
{
    if (!h || !ws) return fail(MOE_ERR_INVALID_ARG, "moe_get_indices: NULL handle or workspace");
    const WsLayout L = layout_of(h, T_cap);
    const char* w = (const char*)ws;
    WsHeader hdr;
    hipError_t e = hipMemcpyAsync(&hdr, w + L.hdr, sizeof(hdr), hipMemcpyDeviceToHost, stream);
    if (e == hipSuccess) e = hipStreamSynchronize(stream);
    if (e != hipSuccess) return hip_fail(e, "moe_get_indices: header copy");
    const int64_t R = (int64_t)hdr.T * h->k;
    if (counts) e = hipMemcpy(counts, w + L.counts, 4 * h->E, hipMemcpyDeviceToHost);
    if (e == hipSuccess && offsets)
        e = hipMemcpy(offsets, w + L.offsets, 4 * (h->E + 1), hipMemcpyDeviceToHost);
    if (e == hipSuccess && perm_src && hdr.n_rows > 0)
        e = hipMemcpy(perm_src, w + L.perm_src, 4 * (size_t)hdr.n_rows, hipMemcpyDeviceToHost);
    if (e == hipSuccess && dst && R > 0)
        e = hipMemcpy(dst, w + L.dst, 4 * (size_t)R, hipMemcpyDeviceToHost);
    if (e != hipSuccess) return hip_fail(e, "moe_get_indices: copy");
    if (n_rows_out) *n_rows_out = hdr.n_rows;
    if (T_out) *T_out = hdr.T;
    return MOE_OK;
}

moe_status moe_get_rows(moe_handle h, const void* ws, int64_t T_cap, float* fc2_rows,
                        void* fc1_out_rows, int32_t* sorted_ids, float* sorted_probs,
                        void* x_codes, void* x_scales, hipStream_t stream)
{
    if (!h || !ws) return fail(MOE_ERR_INVALID_ARG, "moe_get_rows: NULL handle or workspace");
    if ((x_codes || x_scales) && h->precision == MOE_BF16)
        return fail(MOE_ERR_INVALID_ARG, "moe_get_rows: bf16 has no quantized activations");
    const WsLayout L = layout_of(h, T_cap);
    const char* w = (const char*)ws;
    WsHeader hdr;
    hipError_t e = hipMemcpyAsync(&hdr, w + L.hdr, sizeof(hdr), hipMemcpyDeviceToHost, stream);
    if (e == hipSuccess) e = hipStreamSynchronize(stream);
    if (e != hipSuccess) return hip_fail(e, "moe_get_rows: header copy");
    const size_t n = (size_t)hdr.n_rows;
    const size_t T = (size_t)hdr.T;
    const size_t R = T * h->k;
    if (fc2_rows && n) e = hipMemcpy(fc2_rows, w + L.obuf, 4 * n * h->H, hipMemcpyDeviceToHost);
    if (e == hipSuccess && fc1_out_rows && n) {
        if (h->precision == MOE_BF16) {
            e = hipMemcpy(fc1_out_rows, w + L.hbuf, 2 * n * h->F, hipMemcpyDeviceToHost);
        } else {
            e = hipMemcpy(fc1_out_rows, w + L.hbuf, n * h->F, hipMemcpyDeviceToHost);
            if (e == hipSuccess)
                e = hipMemcpy((char*)fc1_out_rows + n * h->F, w + L.hscale, n * (h->F / 32),
                              hipMemcpyDeviceToHost);
        }
    }
    if (e == hipSuccess && sorted_ids && R)
        e = hipMemcpy(sorted_ids, w + L.sorted_ids, 4 * R, hipMemcpyDeviceToHost);
    if (e == hipSuccess && sorted_probs && R)
        e = hipMemcpy(sorted_probs, w + L.sorted_probs, 4 * R, hipMemcpyDeviceToHost);
    if (e == hipSuccess && x_codes && T)
        e = hipMemcpy(x_codes, w + L.xq, T * h->H, hipMemcpyDeviceToHost);
    if (e == hipSuccess && x_scales && T)
        e = hipMemcpy(x_scales, w + L.xs, T * (h->H / 32), hipMemcpyDeviceToHost);
    if (e != hipSuccess) return hip_fail(e, "moe_get_rows: copy");
    return MOE_OK;
}

moe_status moe_set_stage_events(moe_handle h, hipEvent_t* events, int n_events)
{
    if (!h) return fail(MOE_ERR_INVALID_ARG, "moe_set_stage_events: NULL handle");
    if (!events) { h->record_stages = false; return MOE_OK; }
    if (n_events != 6) return fail(MOE_ERR_INVALID_ARG, "moe_set_stage_events: n_events must be 6");
    for (int i = 0; i < 6; ++i) h->stage_events[i] = events[i];
    h->record_stages = true;
    return MOE_OK;
}

moe_status moe_check(moe_handle h, void* ws, hipStream_t stream, uint32_t* err_bits)
{
    if (!h || !ws || !err_bits) return fail(MOE_ERR_INVALID_ARG, "moe_check: NULL argument");
    uint32_t word = 0;
    hipError_t e = hipMemcpyAsync(&word, ws, sizeof(word), hipMemcpyDeviceToHost, stream);
    if (e == hipSuccess) e = hipStreamSynchronize(stream);
    if (e != hipSuccess) return hip_fail(e, "moe_check: read");
    *err_bits = word;
    const uint32_t zero = 0;
    e = hipMemcpyAsync(ws, &zero, sizeof(zero), hipMemcpyHostToDevice, stream);
    if (e == hipSuccess) e = hipStreamSynchronize(stream);
    if (e != hipSuccess) return hip_fail(e, "moe_check: clear");
    if (*err_bits) {
        const uint32_t b = *err_bits;
        return fail(MOE_ERR_DEVICE_CONTRACT, "moe_check: contract violations 0x%x:%s%s%s%s", b,
                    (b & kErrBadId) ? " expert id outside [0, E) (route dropped);" : "",
                    (b & kErrDupId) ? " expert id repeated within a token (repeat dropped);" : "",
                    (b & kErrLiveHigh) ? " live count above capacity (clamped);" : "",
                    (b & kErrLiveNeg) ? " negative live count (taken as 0);" : "");
    }
    return MOE_OK;
}

}  // extern "C"
