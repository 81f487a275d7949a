// C ABI of libtpg_moe.so: host-side argument checks, the workspace layout, and the
// launch sequence of each entry point on the caller's stream.  No entry point
// synchronises, allocates, or reads device memory on the host.
#include <string.h>

#include <mutex>

#include "moe_internal.h"

// Scratch of moe_forward_noalloc: one array per GPU the library runs on (each holds it until the
// process ends).  In host code `scratch` is only a stand-in for the symbol; its device address
// comes from hipGetSymbolAddress, once per device, and only that address is ever used.
static __device__ __align__(256) unsigned char scratch[MOE_NOALLOC_SCRATCH_BYTES];

namespace tpg {

namespace {

thread_local int g_last_hip_error = 0;

size_t align256(size_t x) { return (x + 255) & ~(size_t)255; }

int check_problem(const moe_problem *p) {
    if (!p) return MOE_ERR_NULL;
    if (p->T < 0 || p->E < 1 || p->E > 256 || p->k < 1 || p->k > p->E) return MOE_ERR_SHAPE;
    if (p->H < 128 || p->H > 65536 || p->H % 128 != 0) return MOE_ERR_SHAPE;
    if (p->I < 128 || p->I > 65536 || p->I % 128 != 0) return MOE_ERR_SHAPE;
    if ((int64_t)p->T * p->k >= ((int64_t)1 << 31)) return MOE_ERR_SHAPE;
    // one expert matrix must stay below 2 GB (32-bit byte offsets inside a matrix)
    if ((int64_t)p->H * p->I * 4 >= ((int64_t)1 << 31)) return MOE_ERR_SHAPE;
    if (p->prec != MOE_PREC_BF16 && p->prec != MOE_PREC_W4A8 && p->prec != MOE_PREC_W4A8_MX)
        return MOE_ERR_UNSUPPORTED;
    // W4A8 stages K 256 at a time: H and I multiples of 256
    if (p->prec != MOE_PREC_BF16 && (p->H % 256 != 0 || p->I % 256 != 0)) return MOE_ERR_SHAPE;
    if (p->glu_interleave != 0 && p->glu_interleave != 32) return MOE_ERR_UNSUPPORTED;
    if (!(p->swiglu_clamp >= 0.0f) || p->swiglu_clamp > 3.0e38f) return MOE_ERR_UNSUPPORTED;  // also rejects NaN
    // one flag at a time (the single-launch kernel keeps the expert-order y rows)
    if (p->flags != 0 && p->flags != MOE_FLAG_SINGLE_LAUNCH && p->flags != MOE_FLAG_SCATTER_Y)
        return MOE_ERR_UNSUPPORTED;
    return MOE_OK;
}

int hip_status(hipError_t e) {
    if (e == hipSuccess) return MOE_OK;
    g_last_hip_error = (int)e;
    return MOE_ERR_HIP;
}

// fp8 activations with fp4 weights (NVFP4 or MXFP4)
bool is_w4a8(const moe_problem *p) { return p->prec == MOE_PREC_W4A8 || p->prec == MOE_PREC_W4A8_MX; }

int check_weights(const moe_weights *w, const moe_problem *p) {
    if (!w || !w->w1 || !w->w2) return MOE_ERR_NULL;
    if (is_w4a8(p) && (!w->w1_bscale || !w->w1_gscale || !w->w2_bscale || !w->w2_gscale)) return MOE_ERR_NULL;
    if (is_w4a8(p) && w->w4_layout != MOE_W4_LAYOUT_ROWS && w->w4_layout != MOE_W4_LAYOUT_TILED)
        return MOE_ERR_UNSUPPORTED;
    return MOE_OK;
}

}  // namespace

WsLayout ws_layout(const moe_problem &p) {
    WsLayout L;
    const size_t S = (size_t)n_slots(p), E = (size_t)p.E;
    const size_t act = is_w4a8(&p) ? 1 : 2;  // bytes per activation element
    size_t o = 0;
    L.fsync = o;
    if (is_w4a8(&p))
        o = align256(o + sizeof(FusedSync) +
                     4 * kSyncLine * ((size_t)max_m_tiles(p) * (p.I / 128) + (size_t)max_m_tiles(p)));
    L.chunk_counts = o;
    o = align256(o + (size_t)n_chunks(p) * E * 4);
    L.permute_end = o;
    L.tiles = o;
    o = align256(o + (size_t)max_m_tiles(p) * 2 * 4);
    L.n_tiles = o;
    o = align256(o + 16);
    L.h = o;
    o = align256(o + S * (size_t)p.I * act);
    L.h_scale = o;
    if (is_w4a8(&p)) o = align256(o + S * (size_t)(p.I / 128) * 4);
    L.h32 = o;
    if (is_w4a8(&p)) o = align256(o + S * (size_t)p.I * 4 * (w4a8_split_gemm1(p) ? 4 : 1));
    L.ffn_end = o;
    L.topk_idx = o;
    o = align256(o + S * 4);
    L.topk_w = o;
    o = align256(o + S * 4);
    L.offsets = o;
    o = align256(o + (E + 1) * 4);
    L.row_src = o;
    o = align256(o + S * 4);
    L.slot_row = o;
    o = align256(o + S * 4);
    L.x_perm = o;  // the forward gathers inside GEMM1 where the offsets into x fit: no x_perm then
    if (!fused_gather(p)) o = align256(o + S * (size_t)p.H * act);
    L.x_perm_scale = o;
    if (is_w4a8(&p) && !fused_gather(p)) o = align256(o + S * (size_t)(p.H / 128) * 4);
    L.y_perm = o;
    o = align256(o + S * (size_t)p.H * 2);
    L.forward_end = o;
    return L;
}

namespace {

int run_permute(const void *x, const float *x_scale, const int32_t *topk_idx, const moe_problem &p, int32_t *offsets,
                int32_t *row_src, int32_t *slot_row, void *x_perm, float *x_perm_scale, char *ws, hipStream_t s,
                void *const *ev = nullptr) {
    const WsLayout L = ws_layout(p);
    int32_t *chunk_counts = (int32_t *)(ws + L.chunk_counts);
    auto mark = [&](int i) -> int { return ev ? hip_status(hipEventRecord((hipEvent_t)ev[i], s)) : MOE_OK; };
    int st = mark(0);
    if (!st)
        st = hip_status(launch_tables(topk_idx, p.T, p.k, p.E, chunk_counts, offsets, row_src, slot_row, 0, 0, nullptr,
                                      nullptr, s));
    if (!st) st = mark(1);
    if (!st)
        st = hip_status(launch_permute(x, is_w4a8(&p) ? x_scale : nullptr, slot_row, p.T, p.k, p.H,
                                       is_w4a8(&p) ? 1 : 2, x_perm, x_perm_scale, s));
    if (!st) st = mark(2);
    return st;
}

int run_grouped_ffn(const void *x_perm, const float *x_perm_scale, const int32_t *offsets, const moe_weights &w,
                    const moe_problem &p, void *y_perm, char *ws, hipStream_t s) {
    const WsLayout L = ws_layout(p);
    int32_t *tiles = (int32_t *)(ws + L.tiles);
    int32_t *n_tiles = (int32_t *)(ws + L.n_tiles);
    const int64_t max_tiles = max_m_tiles(p);
    int st = hip_status(launch_build_tiles(offsets, p.E, gemm_bm(p), tile_order(p), tiles, n_tiles, s));
    if (st) return st;
    if (is_w4a8(&p))
        return hip_status(launch_grouped_ffn_w4a8((const uint8_t *)x_perm, x_perm_scale, nullptr, offsets, tiles,
                                                  n_tiles, max_tiles, w, p, (float *)(ws + L.h32),
                                                  (uint8_t *)(ws + L.h), (float *)(ws + L.h_scale),
                                                  (uint16_t *)y_perm, nullptr, s));
    uint16_t *h = (uint16_t *)(ws + L.h);
    st = hip_status(launch_gemm1_swiglu_bf16((const uint16_t *)x_perm, (const uint16_t *)w.w1, offsets, tiles,
                                             n_tiles, max_tiles, p.H, p.I, p.glu_interleave, p.swiglu_clamp, h, s));
    if (st) return st;
    return hip_status(launch_gemm2_bf16(h, (const uint16_t *)w.w2, offsets, tiles, n_tiles, max_tiles, p.H, p.I,
                                        (uint16_t *)y_perm, nullptr, s));
}

int forward_impl(const float *logits, const uint8_t *slot_drop, const void *x, const float *x_scale,
                 const moe_weights *w, const moe_problem *p, void *out, void *ws, size_t ws_bytes, hipStream_t stream,
                 void *const *ev) {
    int st = check_problem(p);
    if (st) return st;
    if (p->T == 0) return MOE_OK;
    if (!logits || !x || !out || !ws) return MOE_ERR_NULL;
    if ((st = check_weights(w, p))) return st;
    if (is_w4a8(p) && !x_scale) return MOE_ERR_NULL;
    if (ws_bytes < moe_workspace_bytes(p)) return MOE_ERR_WORKSPACE;
    const WsLayout L = ws_layout(*p);
    char *b = (char *)ws;
    hipStream_t s = stream;
    int32_t *topk_idx = (int32_t *)(b + L.topk_idx);
    float *topk_w = (float *)(b + L.topk_w);
    int32_t *offsets = (int32_t *)(b + L.offsets);
    int32_t *row_src = (int32_t *)(b + L.row_src);
    int32_t *slot_row = (int32_t *)(b + L.slot_row);
    void *x_perm = b + L.x_perm;
    float *x_perm_scale = is_w4a8(p) ? (float *)(b + L.x_perm_scale) : nullptr;
    void *y_perm = b + L.y_perm;
    int32_t *chunk_counts = (int32_t *)(b + L.chunk_counts);
    int32_t *tiles = (int32_t *)(b + L.tiles);
    int32_t *n_tiles = (int32_t *)(b + L.n_tiles);
    const int64_t max_tiles = max_m_tiles(*p);
    auto mark = [&](int i) -> int {
        return ev ? hip_status(hipEventRecord((hipEvent_t)ev[i], s)) : MOE_OK;
    };
    const bool w4 = is_w4a8(p);
    if (p->flags & MOE_FLAG_SINGLE_LAUNCH) {
        if (!w4 || !forward_small_w4a8_fits(*p)) return MOE_ERR_UNSUPPORTED;
        // the whole forward in one launch: its stages have no marks of their own (0-4 before it,
        // 5-7 after it)
        for (int i = 0; i < 5; ++i)
            if ((st = mark(i))) return st;
        char *fs = b + L.fsync;
        if ((st = hip_status(launch_forward_small_w4a8(
                 logits, slot_drop, (const uint8_t *)x, x_scale, *w, *p, max_tiles, (FusedSync *)fs, topk_idx,
                 topk_w, offsets, row_src, slot_row, tiles, n_tiles, (float *)(b + L.h32), (uint8_t *)(b + L.h),
                 (float *)(b + L.h_scale), (uint16_t *)y_perm, (uint16_t *)out, s))))
            return st;
        for (int i = 5; i < 8; ++i)
            if ((st = mark(i))) return st;
        return MOE_OK;
    }
    // up to kChunk slots and 256 tokens (one workgroup routes 64 tokens at a time, four per wave):
    // routing, tables and tile list in one launch (stage marks 1, 2 and the tile-list stage then
    // take no time of their own).  W4A8 layer at T = 64, timed with stage events: 222.6 -> 213.5
    // us; the tiny bf16 layer (T = 64): 53.8 -> 45.9 us
    const bool small = n_slots(*p) <= kChunk && p->T <= 256;
    if ((st = mark(0))) return st;
    if (small) {
        if ((st = hip_status(launch_frontend_small(logits, slot_drop, p->T, p->E, p->k, gemm_bm(*p), tile_order(*p), topk_idx,
                                                   topk_w, offsets, row_src, slot_row, tiles, n_tiles, s))))
            return st;
    } else if ((st = hip_status(launch_route_topk(logits, slot_drop, p->T, p->E, p->k, topk_idx, topk_w, s)))) {
        return st;
    }
    if ((st = mark(1))) return st;
    // the tables' launches (the scan, or tables_small up to 2048 slots) also write the GEMM tile list
    if (!small && (st = hip_status(launch_tables(topk_idx, p->T, p->k, p->E, chunk_counts, offsets, row_src, slot_row,
                                                 gemm_bm(*p), tile_order(*p), tiles, n_tiles, s))))
        return st;
    if ((st = mark(2))) return st;
    const bool fused = fused_gather(*p);
    // scatter epilogue: GEMM2 stores row r at its slot row_src[r], the combine reads slot order
    const bool scatter = (p->flags & MOE_FLAG_SCATTER_Y) != 0;
    const int32_t *row_dst = scatter ? row_src : nullptr;
    if (!fused && (st = hip_status(launch_permute(x, w4 ? x_scale : nullptr, slot_row, p->T, p->k, p->H, w4 ? 1 : 2,
                                                  x_perm, x_perm_scale, s))))
        return st;
    if ((st = mark(3))) return st;
    if ((st = mark(4))) return st;
    if (w4) {
        const uint8_t *a8 = fused ? (const uint8_t *)x : (const uint8_t *)x_perm;
        const float *as = fused ? x_scale : x_perm_scale;
        if ((st = hip_status(launch_grouped_ffn_w4a8(a8, as, fused ? row_src : nullptr, offsets, tiles, n_tiles,
                                                     max_tiles, *w, *p, (float *)(b + L.h32), (uint8_t *)(b + L.h),
                                                     (float *)(b + L.h_scale), (uint16_t *)y_perm, row_dst,
                                                     s))))
            return st;
        if ((st = mark(5))) return st;
    } else {
        uint16_t *h = (uint16_t *)(b + L.h);
        if (fused)
            st = hip_status(launch_gemm1_swiglu_gather_bf16((const uint16_t *)x, row_src, p->T, p->k,
                                                            (const uint16_t *)w->w1, offsets, tiles, n_tiles,
                                                            max_tiles, p->H, p->I, p->glu_interleave,
                                                            p->swiglu_clamp, h, s));
        else
            st = hip_status(launch_gemm1_swiglu_bf16((const uint16_t *)x_perm, (const uint16_t *)w->w1, offsets,
                                                     tiles, n_tiles, max_tiles, p->H, p->I, p->glu_interleave,
                                                     p->swiglu_clamp, h, s));
        if (st) return st;
        if ((st = mark(5))) return st;
        if ((st = hip_status(launch_gemm2_bf16(h, (const uint16_t *)w->w2, offsets, tiles, n_tiles, max_tiles, p->H,
                                               p->I, (uint16_t *)y_perm, row_dst, s))))
            return st;
    }
    if ((st = mark(6))) return st;
    if ((st = hip_status(launch_combine((const uint16_t *)y_perm, slot_row, topk_w, p->T, p->k, p->H, scatter,
                                        (uint16_t *)out, s))))
        return st;
    return mark(7);
}

}  // namespace

}  // namespace tpg

using namespace tpg;

extern "C" {

size_t moe_workspace_bytes(const moe_problem *p) {
    if (check_problem(p) != MOE_OK) return 0;
    return ws_layout(*p).forward_end;
}

size_t moe_call_workspace_bytes(const moe_problem *p, int which) {
    if (check_problem(p) != MOE_OK) return 0;
    const WsLayout L = ws_layout(*p);
    switch (which) {
        case MOE_WS_PERMUTE: return L.permute_end;
        case MOE_WS_GROUPED_FFN: return L.ffn_end;
        case MOE_WS_FORWARD: return L.forward_end;
        default: return 0;
    }
}

const char *moe_status_str(int status) {
    switch (status) {
        case MOE_OK: return "ok";
        case MOE_ERR_NULL: return "a required pointer is NULL";
        case MOE_ERR_SHAPE: return "a problem size is out of range";
        case MOE_ERR_UNSUPPORTED: return "an option value is not supported";
        case MOE_ERR_WORKSPACE: return "workspace is smaller than moe_workspace_bytes()";
        case MOE_ERR_HIP: return "a HIP kernel launch failed";
        case MOE_ERR_SCRATCH:
            return "moe_forward_noalloc: the problem's workspace exceeds the library's 64 MiB scratch "
                   "(use moe_forward with a caller-allocated workspace)";
        default: return "unknown status";
    }
}

int moe_last_hip_error(void) { return g_last_hip_error; }

int moe_route_topk(const float *logits, const uint8_t *slot_drop, const moe_problem *p, int32_t *topk_idx,
                   float *topk_w, hipStream_t stream) {
    int st = check_problem(p);
    if (st) return st;
    if (p->T == 0) return MOE_OK;
    if (!logits || !topk_idx || !topk_w) return MOE_ERR_NULL;
    return hip_status(launch_route_topk(logits, slot_drop, p->T, p->E, p->k, topk_idx, topk_w, stream));
}

int moe_permute(const void *x, const float *x_scale, const int32_t *topk_idx, const moe_problem *p, int32_t *offsets,
                int32_t *row_src, int32_t *slot_row, void *x_perm, float *x_perm_scale, void *ws, size_t ws_bytes,
                hipStream_t stream) {
    int st = check_problem(p);
    if (st) return st;
    if (p->T == 0) return MOE_OK;
    if (!x || !topk_idx || !offsets || !row_src || !slot_row || !x_perm || !ws) return MOE_ERR_NULL;
    if (is_w4a8(p) && (!x_scale || !x_perm_scale)) return MOE_ERR_NULL;
    if (ws_bytes < moe_call_workspace_bytes(p, MOE_WS_PERMUTE)) return MOE_ERR_WORKSPACE;
    return run_permute(x, x_scale, topk_idx, *p, offsets, row_src, slot_row, x_perm, x_perm_scale, (char *)ws,
                       stream);
}

int moe_permute_timed(const void *x, const float *x_scale, const int32_t *topk_idx, const moe_problem *p,
                      int32_t *offsets, int32_t *row_src, int32_t *slot_row, void *x_perm, float *x_perm_scale,
                      void *ws, size_t ws_bytes, hipStream_t stream, void *const *stage_events) {
    if (!stage_events) return MOE_ERR_NULL;
    for (int i = 0; i < MOE_N_PERMUTE_EVENTS; ++i)
        if (!stage_events[i]) return MOE_ERR_NULL;
    int st = check_problem(p);
    if (st) return st;
    if (p->T == 0) return MOE_OK;
    if (!x || !topk_idx || !offsets || !row_src || !slot_row || !x_perm || !ws) return MOE_ERR_NULL;
    if (is_w4a8(p) && (!x_scale || !x_perm_scale)) return MOE_ERR_NULL;
    if (ws_bytes < moe_call_workspace_bytes(p, MOE_WS_PERMUTE)) return MOE_ERR_WORKSPACE;
    return run_permute(x, x_scale, topk_idx, *p, offsets, row_src, slot_row, x_perm, x_perm_scale, (char *)ws,
                       stream, stage_events);
}

int moe_grouped_ffn(const void *x_perm, const float *x_perm_scale, const int32_t *offsets, const moe_weights *w,
                    const moe_problem *p, void *y_perm, void *ws, size_t ws_bytes, hipStream_t stream) {
    int st = check_problem(p);
    if (st) return st;
    if (p->T == 0) return MOE_OK;
    if (!x_perm || !offsets || !y_perm || !ws) return MOE_ERR_NULL;
    if ((st = check_weights(w, p))) return st;
    if (is_w4a8(p) && !x_perm_scale) return MOE_ERR_NULL;
    if (ws_bytes < moe_call_workspace_bytes(p, MOE_WS_GROUPED_FFN)) return MOE_ERR_WORKSPACE;
    return run_grouped_ffn(x_perm, x_perm_scale, offsets, *w, *p, y_perm, (char *)ws, stream);
}

int moe_unpermute_combine(const void *y_perm, const int32_t *slot_row, const float *topk_w, const moe_problem *p,
                          void *out, hipStream_t stream) {
    int st = check_problem(p);
    if (st) return st;
    if (p->T == 0) return MOE_OK;
    if (!y_perm || !slot_row || !topk_w || !out) return MOE_ERR_NULL;
    return hip_status(launch_combine((const uint16_t *)y_perm, slot_row, topk_w, p->T, p->k, p->H, false,
                                     (uint16_t *)out, stream));
}

int moe_forward(const float *logits, const uint8_t *slot_drop, const void *x, const float *x_scale,
                const moe_weights *w, const moe_problem *p, void *out, void *ws, size_t ws_bytes, hipStream_t stream) {
    return forward_impl(logits, slot_drop, x, x_scale, w, p, out, ws, ws_bytes, stream, nullptr);
}

int moe_forward_timed(const float *logits, const uint8_t *slot_drop, const void *x, const float *x_scale,
                      const moe_weights *w, const moe_problem *p, void *out, void *ws, size_t ws_bytes, hipStream_t stream,
                      void *const *stage_events) {
    if (!stage_events) return MOE_ERR_NULL;
    for (int i = 0; i < MOE_N_STAGE_EVENTS; ++i)
        if (!stage_events[i]) return MOE_ERR_NULL;
    return forward_impl(logits, slot_drop, x, x_scale, w, p, out, ws, ws_bytes, stream, stage_events);
}

namespace {
constexpr int kMaxScratchDevices = 256;
std::mutex g_scratch_mu;
void *g_scratch_dev[kMaxScratchDevices];  // device address of `scratch` on each device, once known

// The device address of `scratch` on the device `stream` belongs to (the current device for the
// null stream), looked up on the first call for that device with the device made current.
int scratch_address(hipStream_t stream, void **out) {
    int dev = -1;
    hipError_t e = stream ? hipStreamGetDevice(stream, &dev) : hipGetDevice(&dev);
    if (e != hipSuccess) return hip_status(e);
    if (dev < 0 || dev >= kMaxScratchDevices) return MOE_ERR_UNSUPPORTED;
    std::lock_guard<std::mutex> lock(g_scratch_mu);
    if (!g_scratch_dev[dev]) {
        int cur = -1;
        if ((e = hipGetDevice(&cur)) != hipSuccess) return hip_status(e);
        if (cur != dev && (e = hipSetDevice(dev)) != hipSuccess) return hip_status(e);
        void *ptr = nullptr;
        e = hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch));
        if (cur != dev) {
            const hipError_t back = hipSetDevice(cur);
            if (e == hipSuccess) e = back;
        }
        if (e != hipSuccess) return hip_status(e);
        if (!ptr) return MOE_ERR_HIP;
        g_scratch_dev[dev] = ptr;
    }
    *out = g_scratch_dev[dev];
    return MOE_OK;
}
}  // namespace

int moe_forward_noalloc(const float *logits, const uint8_t *slot_drop, const void *x, const float *x_scale,
                        const moe_weights *w, const moe_problem *p, void *out, hipStream_t stream) {
    int st = check_problem(p);
    if (st) return st;
    if (p->T == 0) return MOE_OK;
    if (ws_layout(*p).forward_end > MOE_NOALLOC_SCRATCH_BYTES) return MOE_ERR_SCRATCH;
    void *ws = nullptr;
    if ((st = scratch_address(stream, &ws))) return st;
    return forward_impl(logits, slot_drop, x, x_scale, w, p, out, ws, MOE_NOALLOC_SCRATCH_BYTES, stream, nullptr);
}

int moe_w4a8_dequant_table(uint8_t *out8, hipStream_t stream) {
    if (!out8) return MOE_ERR_NULL;
    return hip_status(launch_w4a8_dequant_table(out8, stream));
}

int moe_w4a8_tile_weights(const void *codes, const void *bscale, void *codes_tiled, void *bscale_tiled, int32_t E,
                          int32_t N, int32_t K, int32_t prec, hipStream_t stream) {
    if (!codes || !bscale || !codes_tiled || !bscale_tiled) return MOE_ERR_NULL;
    if (prec != MOE_PREC_W4A8 && prec != MOE_PREC_W4A8_MX) return MOE_ERR_UNSUPPORTED;
    if (E < 1 || N < 32 || N % 32 != 0 || K < 256 || K % 256 != 0) return MOE_ERR_SHAPE;
    const bool mx = prec == MOE_PREC_W4A8_MX;
    const uint64_t nc = (uint64_t)E * N * (K / 2), ns = (uint64_t)E * N * (K / (mx ? 32 : 16));
    auto overlap = [](const void *a, uint64_t na, const void *b, uint64_t nb) {
        const uintptr_t x = (uintptr_t)a, y = (uintptr_t)b;
        return x < y + nb && y < x + na;
    };
    if (overlap(codes, nc, codes_tiled, nc) || overlap(bscale, ns, bscale_tiled, ns) ||
        overlap(codes, nc, bscale_tiled, ns) || overlap(bscale, ns, codes_tiled, nc))
        return MOE_ERR_UNSUPPORTED;
    return hip_status(launch_tile_weights((const uint8_t *)codes, (const uint8_t *)bscale, (uint8_t *)codes_tiled,
                                          (uint8_t *)bscale_tiled, E, N, K, mx, stream));
}

}  // extern "C"
