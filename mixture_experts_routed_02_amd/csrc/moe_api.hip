// Host side of libmoe_mi355x.so: argument checks (fail closed, before any
// enqueue), workspace layout, kernel-plan choice and the stream-ordered
// launches of each entry point declared in include/moe_mi355x.h.
#include "../../include/moe_mi355x.h"
#include "moe_internal.h"

#include <mutex>
#include <new>

// Workspace of moe_forward_noalloc: a file-scope device array, one copy per
// GPU the library runs on, held until the process ends.  Host code never uses
// this name as an address (on the host it is only a stand-in for the symbol):
// each device's address comes from hipGetSymbolAddress, taken once per device
// with that device current (scratch_on_current_device below).
constexpr size_t kScratchBytes = size_t(128) << 20;
static __device__ __align__(256) unsigned char scratch[kScratchBytes];

using moe::GemmPlan;
using moe::Shape;

namespace {

constexpr size_t kAlign = 256;

size_t align_up(size_t v) { return (v + kAlign - 1) / kAlign * kAlign; }

bool aligned(const void* p, size_t a) { return ((uintptr_t)p % a) == 0; }

moe_status_t check_problem(const moe_problem_t* p, Shape* s) {
    if (!p) return MOE_ERROR_INVALID_VALUE;
    if (p->num_tokens < 0 || p->top_k < 1 || p->num_experts < 1 || p->hidden <= 0 ||
        p->intermediate <= 0 || p->capacity < 0)
        return MOE_ERROR_INVALID_VALUE;
    if (p->top_k > 64 || p->num_experts > moe::kMaxExperts) return MOE_ERROR_NOT_SUPPORTED;
    if (p->hidden % 64 != 0 || p->intermediate % 64 != 0) return MOE_ERROR_NOT_SUPPORTED;
    if (p->kernel_hint < 0 || p->kernel_hint > moe::kTiledLarge) return MOE_ERROR_INVALID_VALUE;
    const long long tk = (long long)p->num_tokens * p->top_k;
    if (tk > (1ll << 28)) return MOE_ERROR_NOT_SUPPORTED;
    const long long cap = p->capacity ? p->capacity : tk;
    if (cap < tk) return MOE_ERROR_INVALID_VALUE;
    s->T = p->num_tokens;
    s->K = p->top_k;
    s->E = p->num_experts;
    s->H = p->hidden;
    s->I = p->intermediate;
    s->cap = (int)cap;
    return MOE_SUCCESS;
}

// Workspace layout (every region 256-byte aligned):
//   blk_counts int32 [(rows + 1) * E]   (multi-block dispatch or routed counting
//                                        only: per-block histograms, scanned in
//                                        place, + totals)
//   row_src    int32 [cap]        (moe_forward)
//   token_row  int32 [T*K]        (moe_forward)
//   h          bf16  [cap, I]     (expert compute)
//   y_disp     bf16  [cap, H]     (moe_forward)
struct Layout {
    size_t counts, row_src, token_row, h, y, total;
};

Layout layout(const Shape& s) {
    Layout L{};
    // histogram rows: the multi-block dispatch's, or the routed counting's
    const int nblk = moe::dispatch_blocks(s);
    const int rows = nblk > 1 ? nblk : 0;
    const int rrows = moe::route_count_rows(s);
    const int nrows = rows > rrows ? rows : rrows;
    size_t off = 0;
    L.counts = off;
    off += align_up(nrows > 0 ? (size_t)(nrows + 1) * s.E * 4 : 0);
    L.row_src = off;
    off += align_up((size_t)s.cap * 4);
    L.token_row = off;
    off += align_up((size_t)s.T * s.K * 4);
    L.h = off;
    off += align_up((size_t)s.cap * s.I * 2);
    L.y = off;
    off += align_up((size_t)s.cap * s.H * 2);
    L.total = off;
    return L;
}

template <typename T>
T* at(void* ws, size_t off) {
    return reinterpret_cast<T*>(static_cast<char*>(ws) + off);
}

moe_status_t launched(hipError_t e) { return e == hipSuccess ? MOE_SUCCESS : MOE_ERROR_LAUNCH; }

// A pointer is acceptable if it is aligned and non-null, or null for an
// empty tensor (T = 0).
bool bad_bf16(const void* p, long long n = 1) { return p ? !aligned(p, 16) : n != 0; }
bool bad_i32(const void* p, long long n = 1) { return p ? !aligned(p, 4) : n != 0; }

moe_status_t check_ws(const Shape& s, const void* ws, size_t ws_bytes) {
    if (!ws || !aligned(ws, 16)) return MOE_ERROR_INVALID_VALUE;
    if (ws_bytes < layout(s).total) return MOE_ERROR_INVALID_VALUE;
    return MOE_SUCCESS;
}

moe_status_t expert_compute_impl(const Shape& s, const GemmPlan& plan, const uint16_t* a,
                                 const int32_t* row_src, const int32_t* offsets,
                                 const uint16_t* wgu, const uint16_t* wd, uint16_t* h,
                                 uint16_t* y, hipStream_t st, bool tiled_packed = false) {
    hipError_t e = moe::launch_grouped_gemm(s, plan, true, a, row_src, s.K, offsets, wgu, h, s.H,
                                            s.I, st, tiled_packed);
    if (e != hipSuccess) return MOE_ERROR_LAUNCH;
    e = moe::launch_grouped_gemm(s, plan, false, h, nullptr, 1, offsets, wd, y, s.I, s.H, st,
                                 tiled_packed);
    return launched(e);
}

// Plan for weights in the tiled pack layout: a tiled plan (hint 2..4, or the
// automatic choice with the skinny plan replaced by the 64-row tiled one).
bool tiled_plan(const moe_problem_t* p, const Shape& s, GemmPlan* plan) {
    if (p->kernel_hint == moe::kSkinny) return false;
    *plan = moe::choose_plan(s, p->kernel_hint);
    if (plan->kind == moe::kSkinny) *plan = moe::choose_plan(s, moe::kTiled64);
    return true;
}

// Everything moe_forward checks except the workspace.
moe_status_t check_forward_ptrs(const moe_problem_t* p, Shape* s, const uint16_t* x,
                                const int32_t* ids, const float* w, const uint16_t* wgu,
                                const uint16_t* wd, const int32_t* ntok, const int32_t* offsets,
                                const uint16_t* out) {
    moe_status_t st = check_problem(p, s);
    if (st != MOE_SUCCESS) return st;
    const long long tk = (long long)s->T * s->K;
    if (bad_bf16(x, s->T) || bad_i32(ids, tk) || bad_i32(w, tk) || bad_bf16(wgu) ||
        bad_bf16(wd) || bad_i32(offsets) || bad_bf16(out, s->T))
        return MOE_ERROR_INVALID_VALUE;
    if (ntok && !aligned(ntok, 4)) return MOE_ERROR_INVALID_VALUE;
    return MOE_SUCCESS;
}

moe_status_t check_forward_args(const moe_problem_t* p, Shape* s, const uint16_t* x,
                                const int32_t* ids, const float* w, const uint16_t* wgu,
                                const uint16_t* wd, const int32_t* ntok, const int32_t* offsets,
                                const uint16_t* out, const void* ws, size_t ws_bytes) {
    moe_status_t st = check_forward_ptrs(p, s, x, ids, w, wgu, wd, ntok, offsets, out);
    if (st != MOE_SUCCESS) return st;
    return check_ws(*s, ws, ws_bytes);
}

// Device address of `scratch` on the calling thread's current device, looked
// up once per device (the first call there) and kept.
constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices] = {};

moe_status_t scratch_on_current_device(void** ptr) {
    int dev = -1;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return MOE_ERROR_LAUNCH;
    std::lock_guard<std::mutex> lock(g_scratch_mu);
    if (!g_scratch_ptr[dev]) {
        void* p = nullptr;
        if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || !p)
            return MOE_ERROR_LAUNCH;
        g_scratch_ptr[dev] = p;
    }
    *ptr = g_scratch_ptr[dev];
    return MOE_SUCCESS;
}

moe_status_t forward_impl(const Shape& s, int hint, const uint16_t* x, const int32_t* ids,
                          const float* w, const uint16_t* wgu, const uint16_t* wd,
                          const int32_t* ntok, int32_t* offsets, uint16_t* out, void* ws,
                          hipStream_t st) {
    const Layout L = layout(s);
    int32_t* counts = at<int32_t>(ws, L.counts);
    int32_t* row_src = at<int32_t>(ws, L.row_src);
    int32_t* token_row = at<int32_t>(ws, L.token_row);
    uint16_t* h = at<uint16_t>(ws, L.h);
    uint16_t* y = at<uint16_t>(ws, L.y);
    const GemmPlan plan = moe::choose_plan(s, hint);
    if (plan.kind == moe::kSkinny && (long long)s.T * s.K <= moe::kFusedDispatchMax) {
        // small batch: the gate-up kernel does the dispatch itself (one launch fewer)
        if (moe::launch_gateup_fused_dispatch(s, plan, x, ids, ntok, offsets, row_src, token_row,
                                              wgu, h, st) != hipSuccess)
            return MOE_ERROR_LAUNCH;
        if (moe::tiny_down_ok(s))   // tiny batch: the down kernel also combines
            return launched(moe::launch_down_combine_tiny(s, h, offsets, wd, token_row, w, ntok,
                                                          out, st));
        if (moe::launch_grouped_gemm(s, plan, false, h, nullptr, 1, offsets, wd, y, s.I, s.H, st) !=
            hipSuccess)
            return MOE_ERROR_LAUNCH;
    } else {
        if (moe::launch_dispatch(s, ids, ntok, offsets, row_src, token_row, counts, st) !=
            hipSuccess)
            return MOE_ERROR_LAUNCH;
        moe_status_t r = expert_compute_impl(s, plan, x, row_src, offsets, wgu, wd, h, y, st);
        if (r != MOE_SUCCESS) return r;
    }
    if (s.T == 0) return MOE_SUCCESS;
    return launched(moe::launch_combine(s, y, token_row, w, ntok, out, st));
}

// The layer from router logits: the router step fused into the dispatch
// kernels, then expert compute and combine as in forward_impl.
moe_status_t forward_logits_impl(const Shape& s, int hint, int G, const float* logits,
                                 const uint16_t* x, const uint16_t* wgu, const uint16_t* wd,
                                 const int32_t* ntok, int32_t* ids, float* w, int32_t* offsets,
                                 uint16_t* out, void* ws, hipStream_t st) {
    const Layout L = layout(s);
    int32_t* counts = at<int32_t>(ws, L.counts);
    int32_t* row_src = at<int32_t>(ws, L.row_src);
    int32_t* token_row = at<int32_t>(ws, L.token_row);
    uint16_t* h = at<uint16_t>(ws, L.h);
    uint16_t* y = at<uint16_t>(ws, L.y);
    const GemmPlan plan = moe::choose_plan(s, hint);
    if (moe::launch_router_dispatch(s, logits, G, ntok, ids, w, offsets, row_src, token_row,
                                    counts, st) != hipSuccess)
        return MOE_ERROR_LAUNCH;
    if (plan.kind == moe::kSkinny && moe::tiny_down_ok(s)) {
        // tiny batch: gate-up, then the down GEMM with the combine inside
        if (moe::launch_grouped_gemm(s, plan, true, x, row_src, s.K, offsets, wgu, h, s.H, s.I,
                                     st) != hipSuccess)
            return MOE_ERROR_LAUNCH;
        return launched(moe::launch_down_combine_tiny(s, h, offsets, wd, token_row, w, ntok, out,
                                                      st));
    }
    moe_status_t r = expert_compute_impl(s, plan, x, row_src, offsets, wgu, wd, h, y, st);
    if (r != MOE_SUCCESS) return r;
    if (s.T == 0) return MOE_SUCCESS;
    return launched(moe::launch_combine(s, y, token_row, w, ntok, out, st));
}

// Router arguments: G router experts (logits [T, G]), K <= G.
moe_status_t check_router(const Shape& s, int32_t G, const float* logits, const int32_t* ids,
                          const float* w) {
    if (G < 1 || G > (1 << 16)) return MOE_ERROR_NOT_SUPPORTED;
    if (s.K > G) return MOE_ERROR_INVALID_VALUE;
    const long long tk = (long long)s.T * s.K;
    if (bad_i32(logits, (long long)s.T * G) || bad_i32(ids, tk) || bad_i32(w, tk))
        return MOE_ERROR_INVALID_VALUE;
    return MOE_SUCCESS;
}

// bf16 weights in the skinny pack layout: the skinny plan for every batch size.
moe_status_t forward_packed_impl(const Shape& s, const uint16_t* x, const int32_t* ids,
                                 const float* w, const uint16_t* wgu, const uint16_t* wd,
                                 const int32_t* ntok, int32_t* offsets, uint16_t* out, void* ws,
                                 hipStream_t st) {
    const Layout L = layout(s);
    int32_t* counts = at<int32_t>(ws, L.counts);
    int32_t* row_src = at<int32_t>(ws, L.row_src);
    int32_t* token_row = at<int32_t>(ws, L.token_row);
    uint16_t* h = at<uint16_t>(ws, L.h);
    uint16_t* y = at<uint16_t>(ws, L.y);
    const GemmPlan plan = moe::choose_plan(s, moe::kSkinny);
    if ((long long)s.T * s.K <= moe::kFusedDispatchMax) {
        if (moe::launch_gateup_fused_dispatch(s, plan, x, ids, ntok, offsets, row_src, token_row,
                                              wgu, h, st, true) != hipSuccess)
            return MOE_ERROR_LAUNCH;
        if (moe::tiny_down_ok(s))
            return launched(moe::launch_down_combine_tiny(s, h, offsets, wd, token_row, w, ntok,
                                                          out, st, true));
    } else {
        if (moe::launch_dispatch(s, ids, ntok, offsets, row_src, token_row, counts, st) !=
            hipSuccess)
            return MOE_ERROR_LAUNCH;
        if (moe::launch_grouped_gemm_packed(s, true, x, row_src, s.K, offsets, wgu, h, s.H, s.I,
                                            st) != hipSuccess)
            return MOE_ERROR_LAUNCH;
    }
    if (moe::launch_grouped_gemm_packed(s, false, h, nullptr, 1, offsets, wd, y, s.I, s.H, st) !=
        hipSuccess)
        return MOE_ERROR_LAUNCH;
    if (s.T == 0) return MOE_SUCCESS;
    return launched(moe::launch_combine(s, y, token_row, w, ntok, out, st));
}

// MX expert weights (fmt 8 = MXFP8, 4 = MXFP4): the skinny kernels for every
// batch size.
bool bad_codes(const void* p) { return !p || !aligned(p, 16); }
bool bad_scales(const void* p, int fmt) { return !p || !aligned(p, fmt == 8 ? 2 : 4); }

moe_status_t check_mx_problem(const moe_problem_t* p, int fmt, Shape* s, bool packed = false) {
    moe_status_t st = check_problem(p, s);
    if (st != MOE_SUCCESS) return st;
    // packed codes: the skinny kernels only
    if (packed && p->kernel_hint != 0 && p->kernel_hint != moe::kSkinny) return MOE_ERROR_NOT_SUPPORTED;
    if (fmt == 4 && (s->H % 128 != 0 || s->I % 128 != 0)) return MOE_ERROR_NOT_SUPPORTED;
    return MOE_SUCCESS;
}

moe_status_t forward_mx_impl(const Shape& s, int fmt, const uint16_t* x, const int32_t* ids,
                             const float* w, const uint8_t* qgu, const uint8_t* sgu,
                             const uint8_t* qd, const uint8_t* sd, const int32_t* ntok,
                             int32_t* offsets, uint16_t* out, void* ws, hipStream_t st,
                             bool packed, int hint) {
    const Layout L = layout(s);
    int32_t* counts = at<int32_t>(ws, L.counts);
    int32_t* row_src = at<int32_t>(ws, L.row_src);
    int32_t* token_row = at<int32_t>(ws, L.token_row);
    uint16_t* h = at<uint16_t>(ws, L.h);
    uint16_t* y = at<uint16_t>(ws, L.y);
    const bool skinny = packed || moe::choose_plan(s, hint).kind == moe::kSkinny;
    if (skinny && (long long)s.T * s.K <= moe::kFusedDispatchMax) {
        if (moe::launch_gateup_fused_dispatch_mx(s, fmt, x, ids, ntok, offsets, row_src, token_row,
                                                 qgu, sgu, h, st, packed) != hipSuccess)
            return MOE_ERROR_LAUNCH;
        if (moe::tiny_down_ok(s))
            return launched(moe::launch_down_combine_tiny_mx(s, fmt, h, offsets, qd, sd, token_row,
                                                             w, ntok, out, st, packed));
    } else {
        if (moe::launch_dispatch(s, ids, ntok, offsets, row_src, token_row, counts, st) !=
            hipSuccess)
            return MOE_ERROR_LAUNCH;
        if (moe::launch_grouped_gemm_mx(s, fmt, true, x, row_src, s.K, offsets, qgu, sgu, h, s.H,
                                        s.I, st, packed, hint) != hipSuccess)
            return MOE_ERROR_LAUNCH;
    }
    if (moe::launch_grouped_gemm_mx(s, fmt, false, h, nullptr, 1, offsets, qd, sd, y, s.I, s.H,
                                    st, packed, hint) != hipSuccess)
        return MOE_ERROR_LAUNCH;
    if (s.T == 0) return MOE_SUCCESS;
    return launched(moe::launch_combine(s, y, token_row, w, ntok, out, st));
}

moe_status_t check_mx_rows(const void* a, const void* b, int64_t rows, int32_t k) {
    if (rows < 0 || k <= 0 || k % 32 != 0) return MOE_ERROR_INVALID_VALUE;
    if (rows > (1ll << 40) / k) return MOE_ERROR_NOT_SUPPORTED;
    if (rows == 0) return MOE_SUCCESS;
    if (!a || !b || !aligned(a, 16)) return MOE_ERROR_INVALID_VALUE;
    return MOE_SUCCESS;
}

moe_status_t mx_quantize(int fmt, const uint16_t* w, int64_t rows, int32_t k, uint8_t* codes,
                         uint8_t* scales, void* stream) {
    moe_status_t st = check_mx_rows(w, scales, rows, k);
    if (st != MOE_SUCCESS) return st;
    if (rows == 0) return MOE_SUCCESS;
    if (!codes || !aligned(codes, 16)) return MOE_ERROR_INVALID_VALUE;
    return launched(moe::launch_mx_quantize(fmt, w, rows * (k / 32), codes, scales,
                                            static_cast<hipStream_t>(stream)));
}

moe_status_t mx_dequantize(int fmt, const uint8_t* codes, const uint8_t* scales, int64_t rows,
                           int32_t k, uint16_t* w, void* stream) {
    moe_status_t st = check_mx_rows(codes, scales, rows, k);
    if (st != MOE_SUCCESS) return st;
    if (rows == 0) return MOE_SUCCESS;
    if (!w || !aligned(w, 16)) return MOE_ERROR_INVALID_VALUE;
    return launched(moe::launch_mx_dequantize(fmt, codes, scales, rows * (k / 32), w,
                                              static_cast<hipStream_t>(stream)));
}

moe_status_t gate_up_mx(int fmt, const moe_problem_t* p, const uint16_t* x_disp,
                        const int32_t* expert_offsets, const uint8_t* codes, const uint8_t* scales,
                        uint16_t* h, void* stream, bool packed = false) {
    Shape s;
    moe_status_t st = check_mx_problem(p, fmt, &s, packed);
    if (st != MOE_SUCCESS) return st;
    if (bad_bf16(x_disp, s.cap) || bad_i32(expert_offsets) || bad_codes(codes) ||
        bad_scales(scales, fmt) || bad_bf16(h, s.cap))
        return MOE_ERROR_INVALID_VALUE;
    return launched(moe::launch_grouped_gemm_mx(s, fmt, true, x_disp, nullptr, s.K,
                                                expert_offsets, codes, scales, h, s.H, s.I,
                                                static_cast<hipStream_t>(stream), packed,
                                                p->kernel_hint));
}

moe_status_t forward_mx(int fmt, const moe_problem_t* p, const uint16_t* x,
                        const int32_t* topk_ids, const float* topk_weights, const uint8_t* qgu,
                        const uint8_t* sgu, const uint8_t* qd, const uint8_t* sd,
                        const int32_t* num_tokens_dev, int32_t* expert_offsets, uint16_t* out,
                        void* workspace, size_t ws_bytes, void* stream, bool packed = false) {
    Shape s;
    moe_status_t st = check_mx_problem(p, fmt, &s, packed);
    if (st != MOE_SUCCESS) return st;
    const long long tk = (long long)s.T * s.K;
    if (bad_bf16(x, s.T) || bad_i32(topk_ids, tk) || bad_i32(topk_weights, tk) ||
        bad_codes(qgu) || bad_scales(sgu, fmt) || bad_codes(qd) || bad_scales(sd, fmt) ||
        bad_i32(expert_offsets) || bad_bf16(out, s.T))
        return MOE_ERROR_INVALID_VALUE;
    if (num_tokens_dev && !aligned(num_tokens_dev, 4)) return MOE_ERROR_INVALID_VALUE;
    if ((st = check_ws(s, workspace, ws_bytes)) != MOE_SUCCESS) return st;
    return forward_mx_impl(s, fmt, x, topk_ids, topk_weights, qgu, sgu, qd, sd, num_tokens_dev,
                           expert_offsets, out, workspace, static_cast<hipStream_t>(stream),
                           packed, p->kernel_hint);
}

struct GraphHandle {
    hipGraphExec_t exec;
};

}  // namespace

extern "C" {

const char* moe_status_string(moe_status_t status) {
    switch (status) {
        case MOE_SUCCESS: return "MOE_SUCCESS";
        case MOE_ERROR_INVALID_VALUE: return "MOE_ERROR_INVALID_VALUE: bad argument (null/misaligned pointer, size out of range, capacity < T*K, workspace too small)";
        case MOE_ERROR_NOT_SUPPORTED: return "MOE_ERROR_NOT_SUPPORTED: shape outside the supported range (H, I multiples of 64; K <= 64; E <= 512; T*K <= 2^28; moe_forward_noalloc: workspace <= 128 MiB)";
        case MOE_ERROR_LAUNCH: return "MOE_ERROR_LAUNCH: a kernel launch failed";
    }
    return "unknown moe_status_t";
}

moe_status_t moe_workspace_size(const moe_problem_t* p, size_t* bytes) {
    Shape s;
    moe_status_t st = check_problem(p, &s);
    if (st != MOE_SUCCESS) return st;
    if (!bytes) return MOE_ERROR_INVALID_VALUE;
    *bytes = layout(s).total;
    return MOE_SUCCESS;
}

moe_status_t moe_dispatch(const moe_problem_t* p, const uint16_t* x, const int32_t* topk_ids,
                          const int32_t* num_tokens_dev, uint16_t* x_disp,
                          int32_t* expert_offsets, int32_t* row_src, int32_t* token_row,
                          void* workspace, size_t ws_bytes, void* stream) {
    Shape s;
    moe_status_t st = check_problem(p, &s);
    if (st != MOE_SUCCESS) return st;
    const long long tk = (long long)s.T * s.K;
    if (bad_bf16(x, s.T) || bad_i32(topk_ids, tk) || bad_bf16(x_disp, s.cap) ||
        bad_i32(expert_offsets) || bad_i32(row_src, s.cap) || bad_i32(token_row, tk))
        return MOE_ERROR_INVALID_VALUE;
    if (num_tokens_dev && !aligned(num_tokens_dev, 4)) return MOE_ERROR_INVALID_VALUE;
    if ((st = check_ws(s, workspace, ws_bytes)) != MOE_SUCCESS) return st;
    hipStream_t hs = static_cast<hipStream_t>(stream);
    int32_t* counts = at<int32_t>(workspace, layout(s).counts);
    if (moe::launch_dispatch(s, topk_ids, num_tokens_dev, expert_offsets, row_src, token_row,
                             counts, hs) != hipSuccess)
        return MOE_ERROR_LAUNCH;
    return launched(moe::launch_gather(s, x, expert_offsets, row_src, x_disp, hs));
}

moe_status_t moe_expert_compute(const moe_problem_t* p, const uint16_t* x_disp,
                                const int32_t* expert_offsets, const uint16_t* w_gateup,
                                const uint16_t* w_down, uint16_t* y_disp, void* workspace,
                                size_t ws_bytes, void* stream) {
    Shape s;
    moe_status_t st = check_problem(p, &s);
    if (st != MOE_SUCCESS) return st;
    if (bad_bf16(x_disp, s.cap) || bad_i32(expert_offsets) || bad_bf16(w_gateup) ||
        bad_bf16(w_down) || bad_bf16(y_disp, s.cap))
        return MOE_ERROR_INVALID_VALUE;
    if ((st = check_ws(s, workspace, ws_bytes)) != MOE_SUCCESS) return st;
    const GemmPlan plan = moe::choose_plan(s, p->kernel_hint);
    uint16_t* h = at<uint16_t>(workspace, layout(s).h);
    return expert_compute_impl(s, plan, x_disp, nullptr, expert_offsets, w_gateup, w_down, h,
                               y_disp, static_cast<hipStream_t>(stream));
}

moe_status_t moe_gate_up(const moe_problem_t* p, const uint16_t* x_disp,
                         const int32_t* expert_offsets, const uint16_t* w_gateup, uint16_t* h,
                         void* stream) {
    Shape s;
    moe_status_t st = check_problem(p, &s);
    if (st != MOE_SUCCESS) return st;
    if (bad_bf16(x_disp, s.cap) || bad_i32(expert_offsets) || bad_bf16(w_gateup) ||
        bad_bf16(h, s.cap))
        return MOE_ERROR_INVALID_VALUE;
    const GemmPlan plan = moe::choose_plan(s, p->kernel_hint);
    return launched(moe::launch_grouped_gemm(s, plan, true, x_disp, nullptr, s.K, expert_offsets,
                                             w_gateup, h, s.H, s.I,
                                             static_cast<hipStream_t>(stream)));
}

moe_status_t moe_down(const moe_problem_t* p, const uint16_t* h, const int32_t* expert_offsets,
                      const uint16_t* w_down, uint16_t* y_disp, void* stream) {
    Shape s;
    moe_status_t st = check_problem(p, &s);
    if (st != MOE_SUCCESS) return st;
    if (bad_bf16(h, s.cap) || bad_i32(expert_offsets) || bad_bf16(w_down) ||
        bad_bf16(y_disp, s.cap))
        return MOE_ERROR_INVALID_VALUE;
    const GemmPlan plan = moe::choose_plan(s, p->kernel_hint);
    return launched(moe::launch_grouped_gemm(s, plan, false, h, nullptr, 1, expert_offsets,
                                             w_down, y_disp, s.I, s.H,
                                             static_cast<hipStream_t>(stream)));
}

moe_status_t moe_combine(const moe_problem_t* p, const uint16_t* y_disp, const int32_t* token_row,
                         const float* topk_weights, const int32_t* num_tokens_dev, uint16_t* out,
                         void* stream) {
    Shape s;
    moe_status_t st = check_problem(p, &s);
    if (st != MOE_SUCCESS) return st;
    const long long tk = (long long)s.T * s.K;
    if (bad_bf16(y_disp, s.cap) || bad_i32(token_row, tk) || bad_i32(topk_weights, tk) ||
        bad_bf16(out, s.T))
        return MOE_ERROR_INVALID_VALUE;
    if (num_tokens_dev && !aligned(num_tokens_dev, 4)) return MOE_ERROR_INVALID_VALUE;
    if (s.T == 0) return MOE_SUCCESS;
    return launched(moe::launch_combine(s, y_disp, token_row, topk_weights, num_tokens_dev, out,
                                        static_cast<hipStream_t>(stream)));
}

moe_status_t moe_router_topk(const moe_problem_t* p, const float* logits,
                             const int32_t* num_tokens_dev, int32_t* topk_ids,
                             float* topk_weights, void* stream) {
    Shape s;
    moe_status_t st = check_problem(p, &s);
    if (st != MOE_SUCCESS) return st;
    if (s.K > s.E) return MOE_ERROR_INVALID_VALUE;
    const long long tk = (long long)s.T * s.K;
    if (bad_i32(logits, (long long)s.T * s.E) || bad_i32(topk_ids, tk) || bad_i32(topk_weights, tk))
        return MOE_ERROR_INVALID_VALUE;
    if (num_tokens_dev && !aligned(num_tokens_dev, 4)) return MOE_ERROR_INVALID_VALUE;
    if (s.T == 0) return MOE_SUCCESS;
    return launched(moe::launch_router(s, logits, num_tokens_dev, topk_ids, topk_weights,
                                       static_cast<hipStream_t>(stream)));
}

moe_status_t moe_forward(const moe_problem_t* p, const uint16_t* x, const int32_t* topk_ids,
                         const float* topk_weights, const uint16_t* w_gateup,
                         const uint16_t* w_down, const int32_t* num_tokens_dev,
                         int32_t* expert_offsets, uint16_t* out, void* workspace,
                         size_t ws_bytes, void* stream) {
    Shape s;
    moe_status_t st = check_forward_args(p, &s, x, topk_ids, topk_weights, w_gateup, w_down,
                                         num_tokens_dev, expert_offsets, out, workspace, ws_bytes);
    if (st != MOE_SUCCESS) return st;
    return forward_impl(s, p->kernel_hint, x, topk_ids, topk_weights, w_gateup, w_down,
                        num_tokens_dev, expert_offsets, out, workspace,
                        static_cast<hipStream_t>(stream));
}

moe_status_t moe_router_dispatch(const moe_problem_t* p, int32_t router_experts,
                                 const float* logits, const int32_t* num_tokens_dev,
                                 int32_t* topk_ids, float* topk_weights, const uint16_t* x,
                                 uint16_t* x_disp, int32_t* expert_offsets, int32_t* row_src,
                                 int32_t* token_row, void* workspace, size_t ws_bytes,
                                 void* stream) {
    Shape s;
    moe_status_t st = check_problem(p, &s);
    if (st != MOE_SUCCESS) return st;
    if ((st = check_router(s, router_experts, logits, topk_ids, topk_weights)) != MOE_SUCCESS)
        return st;
    const long long tk = (long long)s.T * s.K;
    if (bad_bf16(x, s.T) || bad_bf16(x_disp, s.cap) || bad_i32(expert_offsets) ||
        bad_i32(row_src, s.cap) || bad_i32(token_row, tk))
        return MOE_ERROR_INVALID_VALUE;
    if (num_tokens_dev && !aligned(num_tokens_dev, 4)) return MOE_ERROR_INVALID_VALUE;
    if ((st = check_ws(s, workspace, ws_bytes)) != MOE_SUCCESS) return st;
    hipStream_t hs = static_cast<hipStream_t>(stream);
    int32_t* counts = at<int32_t>(workspace, layout(s).counts);
    if (moe::launch_router_dispatch(s, logits, router_experts, num_tokens_dev, topk_ids,
                                    topk_weights, expert_offsets, row_src, token_row, counts,
                                    hs) != hipSuccess)
        return MOE_ERROR_LAUNCH;
    return launched(moe::launch_gather(s, x, expert_offsets, row_src, x_disp, hs));
}

moe_status_t moe_forward_logits(const moe_problem_t* p, int32_t router_experts,
                                const float* logits, const uint16_t* x, const uint16_t* w_gateup,
                                const uint16_t* w_down, const int32_t* num_tokens_dev,
                                int32_t* topk_ids, float* topk_weights, int32_t* expert_offsets,
                                uint16_t* out, void* workspace, size_t ws_bytes, void* stream) {
    Shape s;
    // topk_ids / topk_weights are outputs here; the shared checks see them as
    // the routing arguments
    moe_status_t st = check_forward_args(p, &s, x, topk_ids, topk_weights, w_gateup, w_down,
                                         num_tokens_dev, expert_offsets, out, workspace, ws_bytes);
    if (st != MOE_SUCCESS) return st;
    if ((st = check_router(s, router_experts, logits, topk_ids, topk_weights)) != MOE_SUCCESS)
        return st;
    return forward_logits_impl(s, p->kernel_hint, router_experts, logits, x, w_gateup, w_down,
                               num_tokens_dev, topk_ids, topk_weights, expert_offsets, out,
                               workspace, static_cast<hipStream_t>(stream));
}

moe_status_t moe_forward_single(const moe_problem_t* p, const uint16_t* x, const int32_t* topk_ids,
                                const float* topk_weights, const uint16_t* w_gateup,
                                const uint16_t* w_down, const int32_t* num_tokens_dev,
                                int32_t* expert_offsets, uint16_t* out, void* workspace,
                                size_t ws_bytes, void* stream) {
    Shape s;
    moe_status_t st = check_forward_args(p, &s, x, topk_ids, topk_weights, w_gateup, w_down,
                                         num_tokens_dev, expert_offsets, out, workspace, ws_bytes);
    if (st != MOE_SUCCESS) return st;
    if (p->kernel_hint > moe::kSkinny || !moe::tiny_down_ok(s) || s.T == 0)
        return MOE_ERROR_NOT_SUPPORTED;
    const Layout L = layout(s);
    const hipError_t e = moe::launch_forward_tiny_single(
        s, x, topk_ids, num_tokens_dev, expert_offsets, at<int32_t>(workspace, L.row_src),
        at<int32_t>(workspace, L.token_row), w_gateup, at<uint16_t>(workspace, L.h), w_down,
        topk_weights, out, static_cast<hipStream_t>(stream));
    if (e == hipErrorCooperativeLaunchTooLarge) return MOE_ERROR_NOT_SUPPORTED;
    return launched(e);
}

moe_status_t moe_single_launch_status(uint32_t* barrier_timeouts) {
    if (!barrier_timeouts) return MOE_ERROR_INVALID_VALUE;
    unsigned int t = 0;
    if (moe::single_launch_status(&t) != hipSuccess) return MOE_ERROR_LAUNCH;
    *barrier_timeouts = t;
    return MOE_SUCCESS;
}

moe_status_t moe_tiled_pack(const uint16_t* w, int32_t experts, int32_t rows, int32_t k,
                            uint16_t* packed, void* stream) {
    if (experts < 0 || rows <= 0 || k <= 0 || rows % 32 != 0 || k % 64 != 0)
        return MOE_ERROR_INVALID_VALUE;
    if ((long long)experts * rows > (1ll << 40) / k) return MOE_ERROR_NOT_SUPPORTED;
    if (experts == 0) return MOE_SUCCESS;
    if (bad_bf16(w) || bad_bf16(packed)) return MOE_ERROR_INVALID_VALUE;
    const uintptr_t n = (uintptr_t)experts * rows * k * 2, a = (uintptr_t)w, b = (uintptr_t)packed;
    if (a < b + n && b < a + n) return MOE_ERROR_INVALID_VALUE;   // overlapping buffers
    return launched(moe::launch_tiled_pack(w, experts, rows, k, packed,
                                           static_cast<hipStream_t>(stream)));
}

moe_status_t moe_gate_up_tiled_packed(const moe_problem_t* p, const uint16_t* x_disp,
                                      const int32_t* expert_offsets,
                                      const uint16_t* w_gateup_packed, uint16_t* h,
                                      void* stream) {
    Shape s;
    moe_status_t st = check_problem(p, &s);
    if (st != MOE_SUCCESS) return st;
    GemmPlan plan;
    if (!tiled_plan(p, s, &plan)) return MOE_ERROR_NOT_SUPPORTED;
    if (bad_bf16(x_disp, s.cap) || bad_i32(expert_offsets) || bad_bf16(w_gateup_packed) ||
        bad_bf16(h, s.cap))
        return MOE_ERROR_INVALID_VALUE;
    return launched(moe::launch_grouped_gemm(s, plan, true, x_disp, nullptr, s.K, expert_offsets,
                                             w_gateup_packed, h, s.H, s.I,
                                             static_cast<hipStream_t>(stream), true));
}

moe_status_t moe_forward_tiled_packed(const moe_problem_t* p, const uint16_t* x,
                                      const int32_t* topk_ids, const float* topk_weights,
                                      const uint16_t* w_gateup_packed,
                                      const uint16_t* w_down_packed,
                                      const int32_t* num_tokens_dev, int32_t* expert_offsets,
                                      uint16_t* out, void* workspace, size_t ws_bytes,
                                      void* stream) {
    Shape s;
    moe_status_t st = check_forward_args(p, &s, x, topk_ids, topk_weights, w_gateup_packed,
                                         w_down_packed, num_tokens_dev, expert_offsets, out,
                                         workspace, ws_bytes);
    if (st != MOE_SUCCESS) return st;
    GemmPlan plan;
    if (!tiled_plan(p, s, &plan)) return MOE_ERROR_NOT_SUPPORTED;
    hipStream_t hs = static_cast<hipStream_t>(stream);
    const Layout L = layout(s);
    int32_t* row_src = at<int32_t>(workspace, L.row_src);
    int32_t* token_row = at<int32_t>(workspace, L.token_row);
    if (moe::launch_dispatch(s, topk_ids, num_tokens_dev, expert_offsets, row_src, token_row,
                             at<int32_t>(workspace, L.counts), hs) != hipSuccess)
        return MOE_ERROR_LAUNCH;
    st = expert_compute_impl(s, plan, x, row_src, expert_offsets, w_gateup_packed, w_down_packed,
                             at<uint16_t>(workspace, L.h), at<uint16_t>(workspace, L.y), hs, true);
    if (st != MOE_SUCCESS) return st;
    if (s.T == 0) return MOE_SUCCESS;
    return launched(moe::launch_combine(s, at<uint16_t>(workspace, L.y), token_row, topk_weights,
                                        num_tokens_dev, out, hs));
}

moe_status_t moe_forward_noalloc(const moe_problem_t* p, const uint16_t* x,
                                 const int32_t* topk_ids, const float* topk_weights,
                                 const uint16_t* w_gateup, const uint16_t* w_down,
                                 const int32_t* num_tokens_dev, int32_t* expert_offsets,
                                 uint16_t* out, void* stream) {
    Shape s;
    moe_status_t st = check_forward_ptrs(p, &s, x, topk_ids, topk_weights, w_gateup, w_down,
                                         num_tokens_dev, expert_offsets, out);
    if (st != MOE_SUCCESS) return st;
    if (layout(s).total > kScratchBytes) return MOE_ERROR_NOT_SUPPORTED;
    void* ws = nullptr;
    if ((st = scratch_on_current_device(&ws)) != MOE_SUCCESS) return st;
    // the workspace regions are written before they are read on every call,
    // so nothing in the shared array needs clearing
    return forward_impl(s, p->kernel_hint, x, topk_ids, topk_weights, w_gateup, w_down,
                        num_tokens_dev, expert_offsets, out, ws, static_cast<hipStream_t>(stream));
}

moe_status_t moe_skinny_pack(const uint16_t* w, int32_t experts, int32_t rows, int32_t k,
                             int32_t gated, uint16_t* packed, void* stream) {
    if (experts < 0 || rows <= 0 || k <= 0 || rows % 16 != 0 || k % 32 != 0 ||
        (gated != 0 && gated != 1))
        return MOE_ERROR_INVALID_VALUE;
    if ((long long)experts * rows > (1ll << 40) / k) return MOE_ERROR_NOT_SUPPORTED;
    if (experts == 0) return MOE_SUCCESS;
    if (bad_bf16(w) || bad_bf16(packed)) return MOE_ERROR_INVALID_VALUE;
    const uintptr_t n = (uintptr_t)experts * rows * k * 2, a = (uintptr_t)w, b = (uintptr_t)packed;
    if (a < b + n && b < a + n) return MOE_ERROR_INVALID_VALUE;   // overlapping buffers
    return launched(moe::launch_skinny_pack(w, experts, rows, k, gated != 0, packed,
                                            static_cast<hipStream_t>(stream)));
}

moe_status_t moe_gate_up_packed(const moe_problem_t* p, const uint16_t* x_disp,
                                const int32_t* expert_offsets, const uint16_t* w_gateup_packed,
                                uint16_t* h, void* stream) {
    Shape s;
    moe_status_t st = check_problem(p, &s);
    if (st != MOE_SUCCESS) return st;
    if (p->kernel_hint != 0 && p->kernel_hint != moe::kSkinny) return MOE_ERROR_NOT_SUPPORTED;
    if (bad_bf16(x_disp, s.cap) || bad_i32(expert_offsets) || bad_bf16(w_gateup_packed) ||
        bad_bf16(h, s.cap))
        return MOE_ERROR_INVALID_VALUE;
    return launched(moe::launch_grouped_gemm_packed(s, true, x_disp, nullptr, s.K, expert_offsets,
                                                    w_gateup_packed, h, s.H, s.I,
                                                    static_cast<hipStream_t>(stream)));
}

moe_status_t moe_forward_packed(const moe_problem_t* p, const uint16_t* x, const int32_t* topk_ids,
                                const float* topk_weights, const uint16_t* w_gateup_packed,
                                const uint16_t* w_down_packed, const int32_t* num_tokens_dev,
                                int32_t* expert_offsets, uint16_t* out, void* workspace,
                                size_t ws_bytes, void* stream) {
    Shape s;
    moe_status_t st = check_forward_args(p, &s, x, topk_ids, topk_weights, w_gateup_packed,
                                         w_down_packed, num_tokens_dev, expert_offsets, out,
                                         workspace, ws_bytes);
    if (st != MOE_SUCCESS) return st;
    if (p->kernel_hint != 0 && p->kernel_hint != moe::kSkinny) return MOE_ERROR_NOT_SUPPORTED;
    return forward_packed_impl(s, x, topk_ids, topk_weights, w_gateup_packed, w_down_packed,
                               num_tokens_dev, expert_offsets, out, workspace,
                               static_cast<hipStream_t>(stream));
}

moe_status_t moe_mxfp8_quantize(const uint16_t* w, int64_t rows, int32_t k, uint8_t* codes,
                                uint8_t* scales, void* stream) {
    return mx_quantize(8, w, rows, k, codes, scales, stream);
}

moe_status_t moe_mxfp8_dequantize(const uint8_t* codes, const uint8_t* scales, int64_t rows,
                                  int32_t k, uint16_t* w, void* stream) {
    return mx_dequantize(8, codes, scales, rows, k, w, stream);
}

moe_status_t moe_gate_up_mxfp8(const moe_problem_t* p, const uint16_t* x_disp,
                               const int32_t* expert_offsets, const uint8_t* w_gateup_codes,
                               const uint8_t* w_gateup_scales, uint16_t* h, void* stream) {
    return gate_up_mx(8, p, x_disp, expert_offsets, w_gateup_codes, w_gateup_scales, h, stream);
}

moe_status_t moe_forward_mxfp8(const moe_problem_t* p, const uint16_t* x, const int32_t* topk_ids,
                               const float* topk_weights, const uint8_t* w_gateup_codes,
                               const uint8_t* w_gateup_scales, const uint8_t* w_down_codes,
                               const uint8_t* w_down_scales, const int32_t* num_tokens_dev,
                               int32_t* expert_offsets, uint16_t* out, void* workspace,
                               size_t ws_bytes, void* stream) {
    return forward_mx(8, p, x, topk_ids, topk_weights, w_gateup_codes, w_gateup_scales,
                      w_down_codes, w_down_scales, num_tokens_dev, expert_offsets, out, workspace,
                      ws_bytes, stream);
}

moe_status_t moe_mxfp4_quantize(const uint16_t* w, int64_t rows, int32_t k, uint8_t* codes,
                                uint8_t* scales, void* stream) {
    return mx_quantize(4, w, rows, k, codes, scales, stream);
}

moe_status_t moe_mxfp4_dequantize(const uint8_t* codes, const uint8_t* scales, int64_t rows,
                                  int32_t k, uint16_t* w, void* stream) {
    return mx_dequantize(4, codes, scales, rows, k, w, stream);
}

moe_status_t moe_gate_up_mxfp4(const moe_problem_t* p, const uint16_t* x_disp,
                               const int32_t* expert_offsets, const uint8_t* w_gateup_codes,
                               const uint8_t* w_gateup_scales, uint16_t* h, void* stream) {
    return gate_up_mx(4, p, x_disp, expert_offsets, w_gateup_codes, w_gateup_scales, h, stream);
}

moe_status_t moe_forward_mxfp4(const moe_problem_t* p, const uint16_t* x, const int32_t* topk_ids,
                               const float* topk_weights, const uint8_t* w_gateup_codes,
                               const uint8_t* w_gateup_scales, const uint8_t* w_down_codes,
                               const uint8_t* w_down_scales, const int32_t* num_tokens_dev,
                               int32_t* expert_offsets, uint16_t* out, void* workspace,
                               size_t ws_bytes, void* stream) {
    return forward_mx(4, p, x, topk_ids, topk_weights, w_gateup_codes, w_gateup_scales,
                      w_down_codes, w_down_scales, num_tokens_dev, expert_offsets, out, workspace,
                      ws_bytes, stream);
}

moe_status_t moe_mx_pack(const uint8_t* codes, int32_t experts, int32_t rows, int32_t k,
                         int32_t bits, int32_t gated, uint8_t* packed, void* stream) {
    if (bits != 8 && bits != 4) return MOE_ERROR_INVALID_VALUE;
    if (k <= 0 || (long long)k * bits % 512 != 0) return MOE_ERROR_INVALID_VALUE;
    // the byte layout of the bf16 pack, on the codes viewed as 16-bit values
    return moe_skinny_pack(reinterpret_cast<const uint16_t*>(codes), experts, rows,
                           (int32_t)((long long)k * bits / 16), gated,
                           reinterpret_cast<uint16_t*>(packed), stream);
}

moe_status_t moe_gate_up_mx_packed(const moe_problem_t* p, int32_t bits, const uint16_t* x_disp,
                                   const int32_t* expert_offsets,
                                   const uint8_t* w_gateup_codes_packed,
                                   const uint8_t* w_gateup_scales, uint16_t* h, void* stream) {
    if (bits != 8 && bits != 4) return MOE_ERROR_INVALID_VALUE;
    return gate_up_mx(bits, p, x_disp, expert_offsets, w_gateup_codes_packed, w_gateup_scales, h,
                      stream, true);
}

moe_status_t moe_forward_mx_packed(const moe_problem_t* p, int32_t bits, const uint16_t* x,
                                   const int32_t* topk_ids, const float* topk_weights,
                                   const uint8_t* w_gateup_codes_packed,
                                   const uint8_t* w_gateup_scales,
                                   const uint8_t* w_down_codes_packed,
                                   const uint8_t* w_down_scales, const int32_t* num_tokens_dev,
                                   int32_t* expert_offsets, uint16_t* out, void* workspace,
                                   size_t ws_bytes, void* stream) {
    if (bits != 8 && bits != 4) return MOE_ERROR_INVALID_VALUE;
    return forward_mx(bits, p, x, topk_ids, topk_weights, w_gateup_codes_packed, w_gateup_scales,
                      w_down_codes_packed, w_down_scales, num_tokens_dev, expert_offsets, out,
                      workspace, ws_bytes, stream, true);
}

moe_status_t moe_mx_tiled_pack(const uint8_t* codes, int32_t experts, int32_t rows, int32_t k,
                               int32_t bits, uint8_t* packed, void* stream) {
    if (bits != 8 && bits != 4) return MOE_ERROR_INVALID_VALUE;
    if (experts < 0 || rows <= 0 || k <= 0 || rows % 32 != 0 || k % 64 != 0)
        return MOE_ERROR_INVALID_VALUE;
    const long long row_bytes = (long long)k * bits / 8;
    if ((long long)experts * rows > (1ll << 40) / row_bytes) return MOE_ERROR_NOT_SUPPORTED;
    if (experts == 0) return MOE_SUCCESS;
    if (bad_codes(codes) || bad_codes(packed)) return MOE_ERROR_INVALID_VALUE;
    const uintptr_t n = (uintptr_t)experts * rows * row_bytes, a = (uintptr_t)codes,
                    b = (uintptr_t)packed;
    if (a < b + n && b < a + n) return MOE_ERROR_INVALID_VALUE;   // overlapping buffers
    return launched(moe::launch_mx_tiled_pack(bits, codes, experts, rows, k, packed,
                                              static_cast<hipStream_t>(stream)));
}

// The tiled plan for codes in the tiled pack layout: as tiled_plan, and both
// GEMMs' K (hidden for gate-up, intermediate for down) within mx_tiled_ok.
static bool mx_tiled_packed_plan(const moe_problem_t* p, const Shape& s, GemmPlan* plan,
                                 bool gate_up_only) {
    if (!tiled_plan(p, s, plan)) return false;
    return moe::mx_tiled_ok(s.H) && (gate_up_only || moe::mx_tiled_ok(s.I));
}

moe_status_t moe_gate_up_mx_tiled_packed(const moe_problem_t* p, int32_t bits,
                                         const uint16_t* x_disp, const int32_t* expert_offsets,
                                         const uint8_t* w_gateup_codes_tiled,
                                         const uint8_t* w_gateup_scales, uint16_t* h,
                                         void* stream) {
    if (bits != 8 && bits != 4) return MOE_ERROR_INVALID_VALUE;
    Shape s;
    moe_status_t st = check_mx_problem(p, bits, &s);
    if (st != MOE_SUCCESS) return st;
    GemmPlan plan;
    if (!mx_tiled_packed_plan(p, s, &plan, true)) return MOE_ERROR_NOT_SUPPORTED;
    if (bad_bf16(x_disp, s.cap) || bad_i32(expert_offsets) || bad_codes(w_gateup_codes_tiled) ||
        bad_scales(w_gateup_scales, bits) || bad_bf16(h, s.cap))
        return MOE_ERROR_INVALID_VALUE;
    return launched(moe::launch_grouped_gemm_mx(s, bits, true, x_disp, nullptr, s.K,
                                                expert_offsets, w_gateup_codes_tiled,
                                                w_gateup_scales, h, s.H, s.I,
                                                static_cast<hipStream_t>(stream), false,
                                                plan.kind, true));
}

moe_status_t moe_forward_mx_tiled_packed(const moe_problem_t* p, int32_t bits, const uint16_t* x,
                                         const int32_t* topk_ids, const float* topk_weights,
                                         const uint8_t* w_gateup_codes_tiled,
                                         const uint8_t* w_gateup_scales,
                                         const uint8_t* w_down_codes_tiled,
                                         const uint8_t* w_down_scales,
                                         const int32_t* num_tokens_dev, int32_t* expert_offsets,
                                         uint16_t* out, void* workspace, size_t ws_bytes,
                                         void* stream) {
    if (bits != 8 && bits != 4) return MOE_ERROR_INVALID_VALUE;
    Shape s;
    moe_status_t st = check_mx_problem(p, bits, &s);
    if (st != MOE_SUCCESS) return st;
    GemmPlan plan;
    if (!mx_tiled_packed_plan(p, s, &plan, false)) return MOE_ERROR_NOT_SUPPORTED;
    const long long tk = (long long)s.T * s.K;
    if (bad_bf16(x, s.T) || bad_i32(topk_ids, tk) || bad_i32(topk_weights, tk) ||
        bad_codes(w_gateup_codes_tiled) || bad_scales(w_gateup_scales, bits) ||
        bad_codes(w_down_codes_tiled) || bad_scales(w_down_scales, bits) ||
        bad_i32(expert_offsets) || bad_bf16(out, s.T))
        return MOE_ERROR_INVALID_VALUE;
    if (num_tokens_dev && !aligned(num_tokens_dev, 4)) return MOE_ERROR_INVALID_VALUE;
    if ((st = check_ws(s, workspace, ws_bytes)) != MOE_SUCCESS) return st;
    hipStream_t hs = static_cast<hipStream_t>(stream);
    const Layout L = layout(s);
    int32_t* row_src = at<int32_t>(workspace, L.row_src);
    int32_t* token_row = at<int32_t>(workspace, L.token_row);
    uint16_t* h = at<uint16_t>(workspace, L.h);
    uint16_t* y = at<uint16_t>(workspace, L.y);
    if (moe::launch_dispatch(s, topk_ids, num_tokens_dev, expert_offsets, row_src, token_row,
                             at<int32_t>(workspace, L.counts), hs) != hipSuccess)
        return MOE_ERROR_LAUNCH;
    if (moe::launch_grouped_gemm_mx(s, bits, true, x, row_src, s.K, expert_offsets,
                                    w_gateup_codes_tiled, w_gateup_scales, h, s.H, s.I, hs, false,
                                    plan.kind, true) != hipSuccess)
        return MOE_ERROR_LAUNCH;
    if (moe::launch_grouped_gemm_mx(s, bits, false, h, nullptr, 1, expert_offsets,
                                    w_down_codes_tiled, w_down_scales, y, s.I, s.H, hs, false,
                                    plan.kind, true) != hipSuccess)
        return MOE_ERROR_LAUNCH;
    if (s.T == 0) return MOE_SUCCESS;
    return launched(moe::launch_combine(s, y, token_row, topk_weights, num_tokens_dev, out, hs));
}

moe_status_t moe_graph_create(const moe_problem_t* p, const uint16_t* x, const int32_t* topk_ids,
                              const float* topk_weights, const uint16_t* w_gateup,
                              const uint16_t* w_down, const int32_t* num_tokens_dev,
                              int32_t* expert_offsets, uint16_t* out, void* workspace,
                              size_t ws_bytes, void** graph_out) {
    Shape s;
    moe_status_t st = check_forward_args(p, &s, x, topk_ids, topk_weights, w_gateup, w_down,
                                         num_tokens_dev, expert_offsets, out, workspace, ws_bytes);
    if (st != MOE_SUCCESS) return st;
    if (!graph_out) return MOE_ERROR_INVALID_VALUE;
    hipStream_t cs = nullptr;
    if (hipStreamCreateWithFlags(&cs, hipStreamNonBlocking) != hipSuccess) return MOE_ERROR_LAUNCH;
    hipGraph_t graph = nullptr;
    moe_status_t r = MOE_SUCCESS;
    if (hipStreamBeginCapture(cs, hipStreamCaptureModeThreadLocal) != hipSuccess) {
        (void)hipStreamDestroy(cs);
        return MOE_ERROR_LAUNCH;
    }
    r = forward_impl(s, p->kernel_hint, x, topk_ids, topk_weights, w_gateup, w_down,
                     num_tokens_dev, expert_offsets, out, workspace, cs);
    hipError_t ec = hipStreamEndCapture(cs, &graph);
    (void)hipStreamDestroy(cs);
    if (r != MOE_SUCCESS || ec != hipSuccess || !graph) {
        if (graph) (void)hipGraphDestroy(graph);
        return MOE_ERROR_LAUNCH;
    }
    hipGraphExec_t exec = nullptr;
    hipError_t ei = hipGraphInstantiate(&exec, graph, nullptr, nullptr, 0);
    (void)hipGraphDestroy(graph);
    if (ei != hipSuccess) return MOE_ERROR_LAUNCH;
    GraphHandle* gh = new (std::nothrow) GraphHandle{exec};
    if (!gh) {
        (void)hipGraphExecDestroy(exec);
        return MOE_ERROR_LAUNCH;
    }
    *graph_out = gh;
    return MOE_SUCCESS;
}

moe_status_t moe_graph_launch(void* graph, void* stream) {
    if (!graph) return MOE_ERROR_INVALID_VALUE;
    GraphHandle* gh = static_cast<GraphHandle*>(graph);
    return launched(hipGraphLaunch(gh->exec, static_cast<hipStream_t>(stream)));
}

moe_status_t moe_graph_destroy(void* graph) {
    if (!graph) return MOE_ERROR_INVALID_VALUE;
    GraphHandle* gh = static_cast<GraphHandle*>(graph);
    (void)hipGraphExecDestroy(gh->exec);
    delete gh;
    return MOE_SUCCESS;
}

}  // extern "C"
