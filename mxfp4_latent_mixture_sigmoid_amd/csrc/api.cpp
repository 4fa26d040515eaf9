// api.cpp -- the C ABI declared in include/mxmoe.h: validation, packed-buffer and workspace
// layouts, and the launch sequence of moe_route / moe_forward on the caller's stream.
#include "kernels.hpp"
#include "mxmoe.h"

#include <climits>
#include <cstdlib>
#include <new>
#include <algorithm>
#include <mutex>
#include <vector>

using namespace mxmoe;

// Workspace of moe_route_forward_static: a file-scope device array, one copy per GPU that the
// library's code object is loaded on, held until the process ends. Host code never passes the
// array's name to a kernel: it uses the device address looked up per device (scratch_address).
static __device__ __align__(256) uint8_t scratch[MOE_STATIC_SCRATCH_BYTES];

struct moe_handle {
    moe_config cfg;
    int Hin;             // width of x and of the router's input
    int E_pad;           // router rows padded to 16
    int E_rx;            // router rows padded to 64 in the combined router + x-side matrix
    uint8_t *packed;
    int64_t off_router, off_xside, off_rx, off_outside, off_gateup, off_down, off_down8, off_gateup4;
    int64_t gateup_stride, down_stride;   // packed bytes per expert
    int64_t off_shared = 0;               // shared gate|up rows on their own (MOE_SHARED_STREAM)
    hipStream_t side = nullptr;           // MOE_SHARED_STREAM: the second stream and its fork/join events
    hipEvent_t fork = nullptr, join = nullptr;
    // profiling hook state
    bool prof = false;
    int prof_max = 0;
    std::vector<int> prof_kid;
    std::vector<hipEvent_t> prof_ev;      // start/stop pairs
};

namespace {

constexpr int64_t ALIGN = 256;
// Expert products: 16-row streaming tiles while experts see few rows (decode), 128-row matrix-core
// tiles once they average TILED_MIN_ROWS rows or more (prefill).
constexpr int BM_STREAM = 16;
constexpr int TILED_MIN_ROWS = 32;
// MOE_SHARED_STREAM with shared experts: their gate|up product runs apart, on the second stream.
bool shared_apart(const moe_config *c)
{
    return c->shared_stream == MOE_SHARED_STREAM && c->has_latent_proj && c->n_shared > 0;
}
// Shared experts whose gate|up columns are part of the x-side product.
int64_t fused_shared(const moe_config *c) { return shared_apart(c) ? 0 : c->n_shared; }
bool tiled_experts(const moe_config *c, int64_t T) { return T * c->top_k >= (int64_t)TILED_MIN_ROWS * c->n_experts; }
int expert_bm(const moe_config *c, int64_t T) { return tiled_experts(c, T) ? TILED_BM : BM_STREAM; }
constexpr int SKINNY_STEPS = 16;   // 32-wide K steps per split of the few-token router product
constexpr int SKINNY_XSTEPS = 16;  // ... and of the few-token x-side and output products
// Few-token x-side and output products: column groups per 512-wide K split (14 x 18 = 252 and
// 9 x 28 = 252 workgroups at K = 7168 and 4352; measured best of 18..72 groups and 512 / 1024-wide
// splits at 64 tokens).
constexpr int XSIDE_GROUPS = 18, OUT_GROUPS = 28;
// ... and of the combined router + x-side product (6016 columns at the full size)
constexpr int RX_GROUPS = 18;

// Router rows in the combined router + x-side matrix: a multiple of the 64-column wave width, so
// that no wave of the many-token product straddles the logits and the z columns.
int64_t router_rows_rx(const moe_config *c) { return ((int64_t)c->n_experts + 63) / 64 * 64; }

int64_t align_up(int64_t v) { return (v + ALIGN - 1) / ALIGN * ALIGN; }

bool valid_config(const moe_config *c)
{
    if (!c)
        return false;
    if (c->act != MOE_ACT_SILU_GLU || (c->has_latent_proj != 0 && c->has_latent_proj != 1))
        return false;
    if (c->stage2 != MOE_STAGE2_BF16 && c->stage2 != MOE_STAGE2_FP8)
        return false;
    if (c->stage1 != MOE_STAGE1_BF16 && c->stage1 != MOE_STAGE1_MXFP4)
        return false;
    if (c->shared_stream != MOE_SHARED_FUSED && c->shared_stream != MOE_SHARED_STREAM)
        return false;
    // the FP8 down product keeps a whole 128-row tile of h (inter bytes per row) in LDS
    if (c->stage2 == MOE_STAGE2_FP8 && (c->inter > FP8_DOWN_MAX_K || c->latent % 64))
        return false;
    if (c->latent <= 0 || c->latent % 128 || c->inter <= 0 || c->inter % 128)
        return false;
    if (c->n_experts < 1 || c->n_experts > 1024 || c->top_k < 1 || c->top_k > 32 || c->top_k > c->n_experts)
        return false;
    if (c->n_shared < 0 || c->n_shared > 8)
        return false;
    if (c->has_latent_proj) {
        if (c->hidden <= 0 || c->hidden % 128)
            return false;
        if (c->n_shared > 0 && (c->shared_inter <= 0 || c->shared_inter % 32))
            return false;
    } else if (c->n_shared != 0) {
        return false;
    }
    // keep every index below 2^31 at T = 0 (sizes are re-checked per call with T)
    const int64_t gateup = (int64_t)c->n_experts * mx_packed_bytes(2 * (int64_t)c->inter, c->latent);
    return gateup > 0;
}

struct PackedLayout {
    int64_t router, xside, rx, outside, shared, gateup, down, down8, gateup4, total, gateup_stride, down_stride;
};

PackedLayout packed_layout(const moe_config *c)
{
    PackedLayout L{};
    const int64_t Hin = c->has_latent_proj ? c->hidden : c->latent;
    const int64_t E_pad = (c->n_experts + 15) / 16 * 16;
    const int64_t Lt = c->latent, H = c->hidden, S = c->n_shared, Is = c->shared_inter, I = c->inter;
    const int64_t Sf = fused_shared(c);
    int64_t off = 0;
    L.router = off;
    off = align_up(off + bf16_packed_bytes(E_pad, Hin));
    L.xside = off;
    if (c->has_latent_proj)
        off = align_up(off + bf16_packed_bytes(Lt + 2 * Sf * Is, H));
    // the router and x-side rows once more as one matrix, for moe_route_forward's single product
    L.rx = off;
    if (c->has_latent_proj)
        off = align_up(off + bf16_packed_bytes(router_rows_rx(c) + Lt + 2 * Sf * Is, H));
    L.outside = off;
    if (c->has_latent_proj)
        off = align_up(off + bf16_packed_bytes(H, Lt + S * Is));
    // MOE_SHARED_STREAM: the shared gate|up rows (16 gate / 16 up alternating) as a matrix of their own
    L.shared = off;
    if (shared_apart(c))
        off = align_up(off + bf16_packed_bytes(2 * S * Is, H));
    L.gateup_stride = mx_packed_bytes(2 * I, Lt);
    L.down_stride = mx_packed_bytes(Lt, I);
    L.gateup = off;
    off = align_up(off + c->n_experts * L.gateup_stride);
    L.down = off;
    off = align_up(off + c->n_experts * L.down_stride);
    // FP8 second stage: the down weights once more, in the scaled instruction's operand layout
    L.down8 = off;
    if (c->stage2 == MOE_STAGE2_FP8)
        off = align_up(off + c->n_experts * L.down_stride);
    // A4W4 first stage: the gate|up weights once more, in the scaled instruction's operand layout
    L.gateup4 = off;
    if (c->stage1 == MOE_STAGE1_MXFP4)
        off = align_up(off + c->n_experts * L.gateup_stride);
    L.total = off;
    return L;
}

struct WsLayout {
    int64_t logits, hist, tiles, z, acat, h, y, h8, z4, partials, total;
    int64_t sync;                       // arrival counter of the few-token top-K launch (T <= SKINNY_MAX_M)
    int64_t rpartials;                  // router partials (inside the partials region, before the dense ones)
    int64_t max_tiles;                  // capacity of the expert tile list (shared by both expert products)
};

int64_t max_tiles(int64_t T, int64_t K, int64_t E, int bm)
{
    const int64_t P = T * K;
    return (P + bm - 1) / bm + (P < E ? P : E);
}

WsLayout ws_layout(const moe_config *c, int64_t T)
{
    WsLayout L{};
    const int64_t E = c->n_experts, K = c->top_k, Lt = c->latent, I = c->inter;
    const int64_t S = c->n_shared, Is = c->shared_inter;
    const int64_t nb = (T + PERM_TOKENS_PER_BLOCK - 1) / PERM_TOKENS_PER_BLOCK;
    L.max_tiles = max_tiles(T, K, E, expert_bm(c, T));
    int64_t off = 0;
    L.logits = off;
    off = align_up(off + T * E * 4);
    L.hist = off;
    off = align_up(off + E * nb * 4);
    L.tiles = off;
    off = align_up(off + (TILE_HEADER_INTS + 4 * L.max_tiles) * 4);
    L.z = off;
    if (c->has_latent_proj)
        off = align_up(off + T * Lt * 2);
    L.acat = off;
    if (c->has_latent_proj)
        off = align_up(off + T * (Lt + S * Is) * 2);
    L.h = off;
    off = align_up(off + T * K * I * 2);
    L.y = off;
    off = align_up(off + T * K * Lt * 2);
    L.h8 = off;   // MX FP8 h: E4M3 codes [T K, I], then E8M0 scales [T K, I / 32]
    if (c->stage2 == MOE_STAGE2_FP8)
        off = align_up(off + T * K * I + T * K * (I / 32));
    L.z4 = off;   // MX FP4 z: E2M1 codes [T, Lt / 2], then E8M0 scales [T, Lt / 32]
    if (c->stage1 == MOE_STAGE1_MXFP4)
        off = align_up(off + T * (Lt / 2) + T * (Lt / 32));
    L.partials = off;
    L.rpartials = off;
    if (T <= SKINNY_MAX_M) {   // split-K partial tiles of the few-token dense products
        // The router's partials and those of the x-side / output products are adjacent, so that
        // the combined router + x-side product of moe_route_forward covers both regions.
        const int64_t Hin = c->has_latent_proj ? c->hidden : c->latent;
        const int64_t Er = c->has_latent_proj ? router_rows_rx(c) : (E + 15) / 16 * 16;
        const int64_t R = SKINNY_MAX_M;   // partial tiles keep 64 rows whatever T is
        off = align_up(off + (int64_t)skinny_splits((int)Hin, SKINNY_STEPS) * R * Er * 4);
        L.partials = off;
        if (c->has_latent_proj) {
            const int64_t H = c->hidden;
            const int64_t p = std::max((int64_t)skinny_splits((int)H, SKINNY_XSTEPS) * R * (Lt + 2 * S * Is),
                                       (int64_t)skinny_splits((int)(Lt + S * Is), SKINNY_XSTEPS) * R * H);
            off = align_up(off + p * 4);
        }
    }
    L.sync = off;
    if (T <= SKINNY_MAX_M)
        off += ALIGN;
    L.total = off;
    return L;
}

// Workspace that serves every T <= T_max. Each region grows with T except the few-token
// split-K partials (present only for T <= SKINNY_MAX_M, at a fixed 64-row size) and the tile
// list (16-row tiles below the tiled-expert threshold, 128-row tiles from there on), so the
// maximum over T <= T_max is reached at T_max, at min(T_max, SKINNY_MAX_M) or just below the
// threshold.
int64_t ws_bytes_upto(const moe_config *c, int64_t T_max)
{
    int64_t best = ws_layout(c, T_max).total;
    best = std::max(best, ws_layout(c, std::min<int64_t>(T_max, SKINNY_MAX_M)).total);
    const int64_t thr = ((int64_t)TILED_MIN_ROWS * c->n_experts + c->top_k - 1) / c->top_k;   // first tiled T
    if (thr - 1 >= 0)
        best = std::max(best, ws_layout(c, std::min(T_max, thr - 1)).total);
    return best;
}

// Largest element index any kernel forms from a 32-bit product must stay below 2^31.
bool sizes_fit_int32(const moe_config *c, int64_t T)
{
    const int64_t P = T * c->top_k;
    return P < INT_MAX && T * c->n_experts < INT_MAX;
}

// Every grid that a call for T tokens launches fits the launch limits (grid.x < 2^31, grid.y <
// 2^16), so that a call that passes argument validation never fails part-way through its
// launches. Mirrors the grid computations of the launchers (rounded up generously).
bool launch_shapes_ok(const moe_config *c, int64_t T)
{
    if (T <= 0)
        return true;
    const int64_t E = c->n_experts, K = c->top_k, Lt = c->latent, I = c->inter, P = T * K;
    const int64_t Hin = c->has_latent_proj ? c->hidden : c->latent;
    const int64_t S = c->has_latent_proj ? c->n_shared : 0, Is = S ? c->shared_inter : 0;
    const int64_t X_MAX = INT32_MAX, Y_MAX = 65535;
    auto cdiv = [](int64_t a, int64_t b) { return (a + b - 1) / b; };
    // dense products (router, x-side, router + x-side, output): the widest output has N columns
    const int64_t N = std::max({(E + 63) / 64 * 64 + Lt + 2 * S * Is, Hin, E + 15});
    if (cdiv(T, TILED_BM) * cdiv(N, 224) + 8 > X_MAX)
        return false;
    // grouping and top-K: one workgroup per 32 tokens / 4 tokens
    if (cdiv(T, 4) > X_MAX)
        return false;
    // expert products over the tile list
    const int64_t tiles = max_tiles(T, K, E, expert_bm(c, T));
    if (!tiled_experts(c, T)) {
        if (tiles > Y_MAX)   // grid.y of the streaming expert kernels
            return false;
    } else {
        const int64_t widest = std::max(cdiv(2 * I, 256), cdiv(Lt, 256));
        if (tiles * widest + 8 > X_MAX)
            return false;
    }
    // quantisers (one thread per eight values), combine (one workgroup per token and 512 columns)
    if (cdiv(P * I / 8, 256) > X_MAX || cdiv(T * Lt / 8, 256) > X_MAX || T * cdiv(Lt, 512) > X_MAX)
        return false;
    return true;
}

bool call_fits(const moe_config *c, int64_t T) { return sizes_fit_int32(c, T) && launch_shapes_ok(c, T); }

bool aligned(const void *p, uintptr_t a) { return ((uintptr_t)p % a) == 0; }

moe_status hip_status(hipError_t e) { return e == hipSuccess ? MOE_OK : MOE_ERR_HIP; }

// Device address of `scratch` on each device, looked up once per device with that device current
// (moe_create's, or the first static call's), then reused.
constexpr int SCRATCH_MAX_DEVICES = 64;
std::mutex scratch_mu;
void *scratch_dev_ptr[SCRATCH_MAX_DEVICES];

moe_status scratch_address(void **out)
{
    int dev = -1;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= SCRATCH_MAX_DEVICES)
        return MOE_ERR_HIP;
    std::lock_guard<std::mutex> lock(scratch_mu);
    if (!scratch_dev_ptr[dev]) {
        void *p = nullptr;
        if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || !p)
            return MOE_ERR_HIP;
        scratch_dev_ptr[dev] = p;
    }
    *out = scratch_dev_ptr[dev];
    return MOE_OK;
}

void prof_mark(moe_handle *h, int kid, hipStream_t st, bool start)
{
    if (!h->prof)
        return;
    if (start) {
        if ((int)h->prof_kid.size() >= h->prof_max)
            return;
        hipEvent_t a = nullptr, b = nullptr;
        if (hipEventCreate(&a) != hipSuccess)
            return;
        if (hipEventCreate(&b) != hipSuccess) {
            (void)hipEventDestroy(a);
            return;
        }
        h->prof_kid.push_back(kid);
        h->prof_ev.push_back(a);
        h->prof_ev.push_back(b);
        (void)hipEventRecord(a, st);
    } else if (!h->prof_kid.empty() && h->prof_kid.back() == kid && h->prof_ev.size() == 2 * h->prof_kid.size()) {
        (void)hipEventRecord(h->prof_ev.back(), st);
    }
}

// Launch `expr` (one or more kernels on `st`), bracketed by profiling events when enabled.
#define MOE_LAUNCH(kid, expr)                                                                                 \
    do {                                                                                                      \
        prof_mark(h, (kid), st, true);                                                                        \
        hipError_t _e = (expr);                                                                               \
        prof_mark(h, (kid), st, false);                                                                       \
        if (_e != hipSuccess)                                                                                 \
            return MOE_ERR_HIP;                                                                               \
    } while (0)


} // namespace

extern "C" {

const char *moe_strerror(moe_status s)
{
    switch (s) {
    case MOE_OK:
        return "success";
    case MOE_ERR_INVALID_ARG:
        return "invalid argument (config, shape, pointer or size)";
    case MOE_ERR_UNSUPPORTED:
        return "unsupported request";
    case MOE_ERR_BUFFER_TOO_SMALL:
        return "packed buffer or workspace too small";
    case MOE_ERR_HIP:
        return "HIP launch or runtime error";
    }
    return "unknown status";
}

moe_status moe_query(const moe_config *cfg, int32_t T_max, size_t *packed_bytes, size_t *workspace_bytes)
{
    if (!valid_config(cfg) || T_max < 0 || !call_fits(cfg, T_max))
        return MOE_ERR_INVALID_ARG;
    if (packed_bytes)
        *packed_bytes = (size_t)packed_layout(cfg).total;
    if (workspace_bytes)
        *workspace_bytes = (size_t)ws_bytes_upto(cfg, T_max);
    return MOE_OK;
}

moe_status moe_query_workspace_layout(const moe_config *cfg, int32_t T, size_t *offsets)
{
    if (!valid_config(cfg) || T < 0 || !call_fits(cfg, T) || !offsets)
        return MOE_ERR_INVALID_ARG;
    const WsLayout W = ws_layout(cfg, T);
    const int64_t v[11] = {W.logits, W.hist, W.tiles, W.z, W.acat, W.h, W.y, W.h8, W.z4, W.rpartials, W.total};
    for (int i = 0; i < 11; i++)
        offsets[i] = (size_t)v[i];
    return MOE_OK;
}

moe_status moe_create(const moe_config *cfg, const moe_weights *w, void *packed, size_t packed_bytes, void *stream,
                      moe_handle **out)
{
    if (!out)
        return MOE_ERR_INVALID_ARG;
    *out = nullptr;
    if (!valid_config(cfg) || !w || !packed || !aligned(packed, ALIGN))
        return MOE_ERR_INVALID_ARG;
    const bool lat = cfg->has_latent_proj != 0, sh = lat && cfg->n_shared > 0;
    const void *need[] = {w->w_router, w->gate_codes, w->gate_scales, w->up_codes, w->up_scales, w->down_codes,
                          w->down_scales};
    for (const void *p : need)
        if (!p)
            return MOE_ERR_INVALID_ARG;
    if (!aligned(w->w_router, 16) || !aligned(w->gate_codes, 4) || !aligned(w->up_codes, 4) ||
        !aligned(w->down_codes, 4))
        return MOE_ERR_INVALID_ARG;
    if (lat && (!w->w_down || !w->w_up || !aligned(w->w_down, 16) || !aligned(w->w_up, 16)))
        return MOE_ERR_INVALID_ARG;
    if (sh && (!w->sh_gate || !w->sh_up || !w->sh_down || !aligned(w->sh_gate, 16) || !aligned(w->sh_up, 16) ||
               !aligned(w->sh_down, 16)))
        return MOE_ERR_INVALID_ARG;
    const PackedLayout L = packed_layout(cfg);
    if (packed_bytes < (size_t)L.total)
        return MOE_ERR_BUFFER_TOO_SMALL;

    moe_handle *h = new (std::nothrow) moe_handle;
    if (!h)
        return MOE_ERR_UNSUPPORTED;
    h->cfg = *cfg;
    h->Hin = lat ? cfg->hidden : cfg->latent;
    h->E_pad = (cfg->n_experts + 15) / 16 * 16;
    h->packed = static_cast<uint8_t *>(packed);
    h->off_router = L.router;
    h->off_xside = L.xside;
    h->off_rx = L.rx;
    h->E_rx = (int)router_rows_rx(cfg);
    h->off_outside = L.outside;
    h->off_shared = L.shared;
    h->off_gateup = L.gateup;
    h->off_down = L.down;
    h->off_down8 = L.down8;
    h->off_gateup4 = L.gateup4;
    h->gateup_stride = L.gateup_stride;
    h->down_stride = L.down_stride;

    hipStream_t st = static_cast<hipStream_t>(stream);
    const int64_t E = cfg->n_experts, Lt = cfg->latent, H = cfg->hidden, I = cfg->inter;
    const int64_t S = sh ? cfg->n_shared : 0, Is = sh ? cfg->shared_inter : 0;
    const int64_t Sf = sh ? fused_shared(cfg) : 0;   // shared experts packed with the x-side rows
    hipError_t e = launch_pack_router(h->packed + L.router, static_cast<const uint16_t *>(w->w_router), E, h->E_pad,
                                      h->Hin, st);
    if (e == hipSuccess && lat)
        e = launch_pack_xside(h->packed + L.xside, static_cast<const uint16_t *>(w->w_down),
                              static_cast<const uint16_t *>(w->sh_gate), static_cast<const uint16_t *>(w->sh_up), Lt,
                              H, Sf, Is, st);
    if (e == hipSuccess && lat)
        e = launch_pack_router_xside(h->packed + L.rx, static_cast<const uint16_t *>(w->w_router), E, h->E_rx,
                                     static_cast<const uint16_t *>(w->w_down), static_cast<const uint16_t *>(w->sh_gate),
                                     static_cast<const uint16_t *>(w->sh_up), Lt, H, Sf, Is, st);
    if (e == hipSuccess && shared_apart(cfg))
        e = launch_pack_xside(h->packed + L.shared, nullptr, static_cast<const uint16_t *>(w->sh_gate),
                              static_cast<const uint16_t *>(w->sh_up), 0, H, S, Is, st);
    if (e == hipSuccess && shared_apart(cfg)) {
        e = hipStreamCreateWithFlags(&h->side, hipStreamNonBlocking);
        if (e == hipSuccess)
            e = hipEventCreateWithFlags(&h->fork, hipEventDisableTiming);
        if (e == hipSuccess)
            e = hipEventCreateWithFlags(&h->join, hipEventDisableTiming);
    }
    if (e == hipSuccess && lat)
        e = launch_pack_outside(h->packed + L.outside, static_cast<const uint16_t *>(w->w_up),
                                static_cast<const uint16_t *>(w->sh_down), Lt, H, S, Is, st);
    if (e == hipSuccess)
        e = launch_pack_gateup(h->packed + L.gateup, static_cast<const uint8_t *>(w->gate_codes),
                               static_cast<const uint8_t *>(w->gate_scales), static_cast<const uint8_t *>(w->up_codes),
                               static_cast<const uint8_t *>(w->up_scales), E, I, Lt, st);
    if (e == hipSuccess)
        e = launch_pack_down(h->packed + L.down, static_cast<const uint8_t *>(w->down_codes),
                             static_cast<const uint8_t *>(w->down_scales), E, I, Lt, st);
    if (e == hipSuccess && cfg->stage1 == MOE_STAGE1_MXFP4)
        e = launch_pack_gateup4(h->packed + L.gateup4, static_cast<const uint8_t *>(w->gate_codes),
                                static_cast<const uint8_t *>(w->gate_scales), static_cast<const uint8_t *>(w->up_codes),
                                static_cast<const uint8_t *>(w->up_scales), E, I, Lt, st);
    if (e == hipSuccess && cfg->stage2 == MOE_STAGE2_FP8)
        e = launch_pack_down8(h->packed + L.down8, static_cast<const uint8_t *>(w->down_codes),
                              static_cast<const uint8_t *>(w->down_scales), E, I, Lt, st);
    if (e != hipSuccess) {
        moe_destroy(h);
        return MOE_ERR_HIP;
    }
    // set-up of moe_route_forward_static's scratch on this device (a failure here is reported by
    // that entry point's first call, which looks the address up again)
    void *scratch_ptr = nullptr;
    (void)scratch_address(&scratch_ptr);
    *out = h;
    return MOE_OK;
}

static void prof_clear(moe_handle *h)
{
    for (hipEvent_t e : h->prof_ev)
        (void)hipEventDestroy(e);
    h->prof_ev.clear();
    h->prof_kid.clear();
    h->prof = false;
}

moe_status moe_profile_begin(moe_handle *h, int32_t max_launches)
{
    if (!h || max_launches <= 0)
        return MOE_ERR_INVALID_ARG;
    prof_clear(h);
    h->prof = true;
    h->prof_max = max_launches;
    try {
        h->prof_kid.reserve(max_launches);
        h->prof_ev.reserve(2 * (size_t)max_launches);
    } catch (...) {
        h->prof = false;
        return MOE_ERR_UNSUPPORTED;
    }
    return MOE_OK;
}

moe_status moe_profile_end(moe_handle *h, int32_t *kernel_ids, float *ms, int32_t *n)
{
    if (!h || !n || *n < 0 || (*n > 0 && (!kernel_ids || !ms)))
        return MOE_ERR_INVALID_ARG;
    moe_status st = MOE_OK;
    const int cap = *n;
    int w = 0;
    for (size_t i = 0; i < h->prof_kid.size() && w < cap; i++) {
        float t = 0.f;
        if (hipEventSynchronize(h->prof_ev[2 * i + 1]) != hipSuccess ||
            hipEventElapsedTime(&t, h->prof_ev[2 * i], h->prof_ev[2 * i + 1]) != hipSuccess) {
            st = MOE_ERR_HIP;
            break;
        }
        kernel_ids[w] = h->prof_kid[i];
        ms[w] = t;
        w++;
    }
    *n = w;
    prof_clear(h);
    return st;
}

void moe_destroy(moe_handle *h)
{
    if (!h)
        return;
    prof_clear(h);
    if (h->join)
        (void)hipEventDestroy(h->join);
    if (h->fork)
        (void)hipEventDestroy(h->fork);
    if (h->side)
        (void)hipStreamDestroy(h->side);
    delete h;
}

} // extern "C"

namespace {

// The grouping by expert runs inside the top-K launch (few tokens, logits from split-K partials):
// the last top-K workgroup writes the routing arrays, and the tile list when `tiles` is set.
void set_grouping(TopkArgs &ta, const moe_routing *r, const WsLayout &W, uint8_t *ws, int32_t *tiles, int bm)
{
    ta.group = 1;
    ta.counts = r->counts;
    ta.offsets = r->offsets;
    ta.sorted_pairs = r->sorted_pairs;
    ta.inv = r->inv;
    ta.tiles = tiles;
    ta.bm = bm;
    ta.arrivals = reinterpret_cast<uint32_t *>(ws + W.sync);
}

// Router product (logits, or split-K partials for few tokens); fills the top-K arguments.
moe_status router_impl(moe_handle *h, const void *x, int32_t T, const float *logit_bias, const float *logits_in,
                       float *logits_out, const moe_routing *r, const WsLayout &W, uint8_t *ws, hipStream_t st,
                       TopkArgs &ta)
{
    const moe_config *c = &h->cfg;
    const int E = c->n_experts, K = c->top_k;
    ta = TopkArgs{};
    ta.T = T;
    ta.E = E;
    ta.K = K;
    ta.ids = r->topk_ids;
    ta.w = r->topk_w;
    ta.splits = 1;
    ta.ld = E;
    if (logits_in) {
        ta.src = logits_in;
    } else if (T <= SKINNY_MAX_M) {   // few tokens: split-K partials, summed (+bias) by the top-K kernel
        float *partials = reinterpret_cast<float *>(ws + W.rpartials);
        const int64_t pstride = (int64_t)(h->E_pad / 16) * SKINNY_TILE_FLOATS;
        // the product also clears the arrival counter of the top-K launch after it
        SkinnyArgs g{static_cast<const uint16_t *>(x), h->Hin, T, h->packed + h->off_router, h->E_pad, h->Hin,
                     partials, pstride, reinterpret_cast<uint32_t *>(ws + W.sync)};
        MOE_LAUNCH(MOE_KERNEL_ROUTER, launch_skinny(g, 4, SKINNY_STEPS, st));
        ta.src = partials;
        ta.partials = 1;
        ta.split_stride = pstride;
        ta.splits = skinny_splits(h->Hin, SKINNY_STEPS);
        ta.bias = logit_bias;
        ta.logits_out = logits_out;
        set_grouping(ta, r, W, ws, nullptr, 0);
    } else {
        float *lg = logits_out ? logits_out : reinterpret_cast<float *>(ws + W.logits);
        GemmArgs g{};
        g.A = static_cast<const uint16_t *>(x);
        g.lda = h->Hin;
        g.B = h->packed + h->off_router;
        g.M = T;
        g.N = h->E_pad;
        g.K = h->Hin;
        g.split = INT_MAX;
        g.lo = OutDesc{OUT_F32, lg, E, 0, E, logit_bias};
        MOE_LAUNCH(MOE_KERNEL_ROUTER, (ring_preferred(g) ? launch_ring(g, st) : launch_tiled(g, false, 0, st)));
        ta.src = lg;
    }
    return MOE_OK;
}

// Top-K -> grouping. With `tiles` set (moe_route_forward), the expert tile lists are built here too,
// from the offsets, so the forward part needs no tile-list launch.
moe_status select_impl(moe_handle *h, int32_t T, const TopkArgs &ta, const moe_routing *r, const WsLayout &W,
                       uint8_t *ws, hipStream_t st, bool tiles)
{
    const moe_config *c = &h->cfg;
    const int E = c->n_experts, K = c->top_k;
    int32_t *tl = reinterpret_cast<int32_t *>(ws + W.tiles);
    const int bm = expert_bm(c, T);
    if (ta.group) {   // grouping (and tile list) inside the top-K launch
        TopkArgs tg = ta;
        tg.tiles = tiles ? tl : nullptr;
        tg.bm = bm;
        MOE_LAUNCH(MOE_KERNEL_TOPK, launch_topk(tg, st));
        return MOE_OK;
    }
    MOE_LAUNCH(MOE_KERNEL_TOPK, launch_topk(ta, st));
    if (T <= PERM_SMALL_MAX_T) {
        MOE_LAUNCH(MOE_KERNEL_PERMUTE, launch_permute_small(r->topk_ids, T, K, E, r->counts, r->offsets,
                                                            r->sorted_pairs, r->inv, st, bm, tiles ? tl : nullptr));
    } else {
        MOE_LAUNCH(MOE_KERNEL_PERMUTE, launch_permute(r->topk_ids, T, K, E, reinterpret_cast<int32_t *>(ws + W.hist),
                                                      r->counts, r->offsets, r->sorted_pairs, r->inv, st, bm,
                                                      tiles ? tl : nullptr));
    }
    return MOE_OK;
}

// MOE_SHARED_STREAM: h_s = bf16(silu(x Wg_s^T) (x Wu_s^T)) into columns Lt.. of [zc | h_s], on the
// handle's second stream, forked off `caller` here; experts_impl joins it back before the output
// product. Few tokens: split-K partials at P (the x-side product's split count and layout), summed
// and gated by the x-side epilogue; many tokens: one product whose epilogue applies the GLU. Each
// element is computed as by the x-side product that holds the shared columns otherwise.
moe_status shared_impl(moe_handle *h, const void *x, int32_t T, uint16_t *Acat, int ldcat, float *P,
                       hipStream_t caller)
{
    const moe_config *c = &h->cfg;
    const int H = c->hidden, Lt = c->latent, Ns = 2 * c->n_shared * c->shared_inter;
    if (hipEventRecord(h->fork, caller) != hipSuccess || hipStreamWaitEvent(h->side, h->fork, 0) != hipSuccess)
        return MOE_ERR_HIP;
    hipStream_t st = h->side;
    if (T <= SKINNY_MAX_M) {
        const int64_t pstride = (int64_t)(Ns / 16) * SKINNY_TILE_FLOATS;
        SkinnyArgs g{static_cast<const uint16_t *>(x), H, T, h->packed + h->off_shared, Ns, H, P, pstride};
        MOE_LAUNCH(MOE_KERNEL_SHARED, launch_skinny_persist(g, 8, XSIDE_GROUPS, SKINNY_XSTEPS, st));
        XsideEpiArgs ea{P, pstride, skinny_splits(H, SKINNY_XSTEPS), T, Ns, 0, Ns, nullptr, Acat + Lt, ldcat,
                        nullptr, c->n_experts, 0, nullptr};
        MOE_LAUNCH(MOE_KERNEL_SHARED, launch_xside_epilogue(ea, st));
    } else {
        GemmArgs g{};
        g.A = static_cast<const uint16_t *>(x);
        g.lda = H;
        g.B = h->packed + h->off_shared;
        g.M = T;
        g.N = Ns;
        g.K = H;
        g.split = INT_MAX;
        g.lo = OutDesc{OUT_GLU, Acat + Lt, ldcat, 0, INT_MAX, nullptr};
        MOE_LAUNCH(MOE_KERNEL_SHARED, (ring_preferred(g) ? launch_ring(g, st) : launch_tiled(g, false, 0, st)));
    }
    return hipEventRecord(h->join, st) == hipSuccess ? MOE_OK : MOE_ERR_HIP;
}

// The x-side products, which need only x: z = bf16(x W_down^T) and h_s = bf16(silu(x Wg_s^T) (x Wu_s^T)).
// With `tiles` set (moe_forward alone) the expert tile lists are built here as well: by the few-token
// epilogue, or by a tile-list launch.
moe_status xside_impl(moe_handle *h, const void *x, int32_t T, const moe_routing *r, const WsLayout &W, uint8_t *ws,
                      hipStream_t st, bool tiles)
{
    const moe_config *c = &h->cfg;
    const bool lat = c->has_latent_proj != 0;
    const int E = c->n_experts, Lt = c->latent, H = c->hidden;
    const int S = lat ? c->n_shared : 0, Is = S ? c->shared_inter : 0;
    const int ldcat = Lt + S * Is, Nx = Lt + 2 * (lat ? (int)fused_shared(c) : 0) * Is;   // x-side columns
    const int bm = expert_bm(c, T);
    uint16_t *Z = reinterpret_cast<uint16_t *>(ws + W.z);
    uint16_t *Acat = reinterpret_cast<uint16_t *>(ws + W.acat);
    int32_t *tl = reinterpret_cast<int32_t *>(ws + W.tiles);
    // MOE_SHARED_STREAM: forked once the x-side product is on the stream, so that it runs beside
    // the routed experts rather than beside that product; its partials follow the product's
    float *ps = lat && T <= SKINNY_MAX_M ? reinterpret_cast<float *>(ws + W.partials) +
                                               (int64_t)skinny_splits(H, SKINNY_XSTEPS) * (Nx / 16) * SKINNY_TILE_FLOATS
                                         : nullptr;
    moe_status e;
    if (lat && T <= SKINNY_MAX_M) {   // z and h_s from split-K partials, summed by the epilogue
        float *partials = reinterpret_cast<float *>(ws + W.partials);
        const int64_t pstride = (int64_t)(Nx / 16) * SKINNY_TILE_FLOATS;
        SkinnyArgs g{static_cast<const uint16_t *>(x), H, T, h->packed + h->off_xside, Nx, H, partials, pstride};
        MOE_LAUNCH(MOE_KERNEL_XSIDE, launch_skinny_persist(g, 8, XSIDE_GROUPS, SKINNY_XSTEPS, st));
        if (shared_apart(c) && (e = shared_impl(h, x, T, Acat, ldcat, ps, st)) != MOE_OK)
            return e;
        XsideEpiArgs ea{partials, pstride, skinny_splits(H, SKINNY_XSTEPS), T, Nx, Lt, Nx - Lt, Z, Acat, ldcat,
                        r->offsets, E, bm, tiles ? tl : nullptr};
        MOE_LAUNCH(MOE_KERNEL_XSIDE_EPI, launch_xside_epilogue(ea, st));
        return MOE_OK;
    }
    if (lat) {   // z and h_s in one pass over x
        GemmArgs g{};
        g.A = static_cast<const uint16_t *>(x);
        g.lda = H;
        g.B = h->packed + h->off_xside;
        g.M = T;
        g.N = Nx;
        g.K = H;
        g.split = Lt;
        g.lo = OutDesc{OUT_BF16, Z, Lt, 0, Lt, nullptr};
        g.hi = OutDesc{OUT_GLU, Acat + Lt, ldcat, Lt, INT_MAX, nullptr};
        MOE_LAUNCH(MOE_KERNEL_XSIDE, (ring_preferred(g) ? launch_ring(g, st) : launch_tiled(g, false, 0, st)));
        if (shared_apart(c) && (e = shared_impl(h, x, T, Acat, ldcat, ps, st)) != MOE_OK)
            return e;
    }
    if (tiles)
        MOE_LAUNCH(MOE_KERNEL_TILEMAP, launch_tilemap(r->offsets, E, bm, tl, st));
    return MOE_OK;
}

// moe_route_forward with the latent projections: the router and the x-side products as one
// product over the combined [router rows (zero-padded to E_rx) | x-side rows] matrix, so that x is
// read once and one launch streams both weight matrices; then top-K and grouping. Few tokens: the
// product leaves split-K partials; one launch sums the router columns' for the top-K and runs the
// x-side epilogue on the rest, and the grouping builds the tile lists. Many tokens: the product's
// epilogue writes the logits (+bias), z and the shared GLU directly, and the grouping builds the
// tile lists.
// Every output element is computed in the same order as by the separate products.
moe_status front_impl(moe_handle *h, const void *x, int32_t T, const float *logit_bias, float *logits_out,
                      const moe_routing *r, const WsLayout &W, uint8_t *ws, hipStream_t st)
{
    const moe_config *c = &h->cfg;
    const int E = c->n_experts, K = c->top_k, Lt = c->latent, H = c->hidden;
    const int S = c->n_shared, Is = S ? c->shared_inter : 0;
    const int ldcat = Lt + S * Is, Nx = Lt + 2 * (int)fused_shared(c) * Is, Erx = h->E_rx, Nrx = Erx + Nx;
    const int bm = expert_bm(c, T);
    uint16_t *Z = reinterpret_cast<uint16_t *>(ws + W.z);
    uint16_t *Acat = reinterpret_cast<uint16_t *>(ws + W.acat);
    // MOE_SHARED_STREAM: forked once the combined product is on the stream (beside the top-K and the
    // routed experts); its partials follow the combined product's
    float *ps = T <= SKINNY_MAX_M ? reinterpret_cast<float *>(ws + W.rpartials) +
                                        (int64_t)skinny_splits(H, SKINNY_XSTEPS) * (Nrx / 16) * SKINNY_TILE_FLOATS
                                  : nullptr;
    moe_status e;
    TopkArgs ta{};
    ta.T = T;
    ta.E = E;
    ta.K = K;
    ta.ids = r->topk_ids;
    ta.w = r->topk_w;
    ta.ld = E;
    if (T <= SKINNY_MAX_M) {
        // the partials of all Nrx columns fill the router's and the x-side's partial regions, which
        // are adjacent in the workspace
        float *P = reinterpret_cast<float *>(ws + W.rpartials);
        const int64_t pstride = (int64_t)(Nrx / 16) * SKINNY_TILE_FLOATS;
        const int splits = skinny_splits(H, SKINNY_XSTEPS);
        // the product also clears the arrival counter of the top-K launch after it
        SkinnyArgs g{static_cast<const uint16_t *>(x), H, T, h->packed + h->off_rx, Nrx, H, P, pstride,
                     reinterpret_cast<uint32_t *>(ws + W.sync)};
        MOE_LAUNCH(MOE_KERNEL_ROUTER_XSIDE, launch_skinny_persist(g, 8, RX_GROUPS, SKINNY_XSTEPS, st));
        if (shared_apart(c) && (e = shared_impl(h, x, T, Acat, ldcat, ps, st)) != MOE_OK)
            return e;
        ta.src = P;
        ta.partials = 1;
        ta.split_stride = pstride;
        ta.splits = splits;
        ta.bias = logit_bias;
        ta.logits_out = logits_out;
        // top-K (with the grouping and the tile lists) and the x-side epilogue in one launch
        set_grouping(ta, r, W, ws, reinterpret_cast<int32_t *>(ws + W.tiles), bm);
        XsideEpiArgs ea{P + (int64_t)(Erx / 16) * SKINNY_TILE_FLOATS, pstride, splits, T, Nx, Lt, Nx - Lt, Z,
                        Acat, ldcat, nullptr, E, bm, nullptr};
        MOE_LAUNCH(MOE_KERNEL_TOPK, launch_topk_xside(ta, ea, st));
        return MOE_OK;
    }
    float *lg = logits_out ? logits_out : reinterpret_cast<float *>(ws + W.logits);
    GemmArgs g{};
    g.A = static_cast<const uint16_t *>(x);
    g.lda = H;
    g.B = h->packed + h->off_rx;
    g.M = T;
    g.N = Nrx;
    g.K = H;
    g.split = Erx;
    g.split2 = Erx + Lt;
    g.lo = OutDesc{OUT_F32, lg, E, 0, E, logit_bias};
    g.hi = OutDesc{OUT_BF16, Z, Lt, Erx, Erx + Lt, nullptr};
    g.top = OutDesc{OUT_GLU, Acat + Lt, ldcat, Erx + Lt, INT_MAX, nullptr};
    MOE_LAUNCH(MOE_KERNEL_ROUTER_XSIDE, (ring_preferred(g) ? launch_ring(g, st) : launch_tiled(g, false, 0, st)));
    if (shared_apart(c) && (e = shared_impl(h, x, T, Acat, ldcat, ps, st)) != MOE_OK)
        return e;
    ta.src = lg;
    ta.splits = 1;
    return select_impl(h, T, ta, r, W, ws, st, true);
}

// Expert products, combine and the output product; needs the routing, the x-side results and the
// tile lists.
moe_status experts_impl(moe_handle *h, const void *x, int32_t T, const moe_routing *r, void *out, const WsLayout &W,
                        uint8_t *ws, hipStream_t st)
{
    const moe_config *c = &h->cfg;
    const bool lat = c->has_latent_proj != 0;
    const int K = c->top_k, Lt = c->latent, I = c->inter, H = c->hidden;
    const int S = lat ? c->n_shared : 0, Is = S ? c->shared_inter : 0;
    const int ldcat = Lt + S * Is;
    uint16_t *Z = reinterpret_cast<uint16_t *>(ws + W.z);
    uint16_t *Acat = reinterpret_cast<uint16_t *>(ws + W.acat);
    uint16_t *Hb = reinterpret_cast<uint16_t *>(ws + W.h);
    uint16_t *Yb = reinterpret_cast<uint16_t *>(ws + W.y);
    int32_t *tl = reinterpret_cast<int32_t *>(ws + W.tiles);
    const bool tiled = tiled_experts(c, T);
    if (c->stage1 == MOE_STAGE1_MXFP4) {   // z -> MX FP4, then h = bf16(silu(g) u) on the scaled instruction
        const uint16_t *A = lat ? Z : static_cast<const uint16_t *>(x);
        uint8_t *zq = ws + W.z4, *zs = ws + W.z4 + (int64_t)T * (Lt / 2);
        MOE_LAUNCH(MOE_KERNEL_Z_QUANT, launch_fp4_quant(A, T, Lt, zq, zs, st));
        A4GateupArgs g{zq, zs, r->sorted_pairs, K, h->packed + h->off_gateup4, h->gateup_stride, 2 * I, Lt, tl, Hb, I};
        MOE_LAUNCH(MOE_KERNEL_GATEUP, tiled ? launch_a4_gateup(g, (int)W.max_tiles, st)
                                            : launch_a4_gateup_small(g, (int)W.max_tiles, st));
    } else {   // h = bf16(silu(z Wg_e^T) (z Wu_e^T)) for every pair, rows in expert-sorted order
        GemmArgs g{};
        g.A = lat ? Z : static_cast<const uint16_t *>(x);
        g.lda = Lt;
        g.a_index = r->sorted_pairs;
        g.a_div = K;
        g.B = h->packed + h->off_gateup;
        g.b_stride = h->gateup_stride;
        g.N = 2 * I;
        g.K = Lt;
        g.tiles = tl;
        g.split = INT_MAX;
        g.lo = OutDesc{OUT_GLU, Hb, I, 0, INT_MAX, nullptr};
        MOE_LAUNCH(MOE_KERNEL_GATEUP, tiled ? launch_tiled(g, true, (int)W.max_tiles, st)
                                            : launch_gemm_grouped(g, (2 * I) % 64 ? GEMM_MX_GLU_M16 : GEMM_MX_GLU_M16_N64,
                                                                  (int)W.max_tiles, st));
    }
    if (c->stage2 == MOE_STAGE2_FP8) {   // h -> MX FP8, then y = bf16(h8 Wd_e^T) on the scaled instruction
        const int64_t P = (int64_t)T * K;
        uint8_t *h8 = ws + W.h8, *h8s = ws + W.h8 + P * I;
        MOE_LAUNCH(MOE_KERNEL_H_QUANT, launch_fp8_quant(Hb, P, I, h8, h8s, st));
        Fp8DownArgs g{h8, h8s, h->packed + h->off_down8, h->down_stride, Lt, I, tl, Yb, Lt};
        MOE_LAUNCH(MOE_KERNEL_DOWN, launch_down_fp8(g, tiled, (int)W.max_tiles, st));
    } else {   // y = bf16(h Wd_e^T), unweighted, expert-sorted rows
        GemmArgs g{};
        g.A = Hb;
        g.lda = I;
        g.B = h->packed + h->off_down;
        g.b_stride = h->down_stride;
        g.N = Lt;
        g.K = I;
        g.tiles = tl;
        g.split = INT_MAX;
        g.lo = OutDesc{OUT_BF16, Yb, Lt, 0, Lt, nullptr};
        MOE_LAUNCH(MOE_KERNEL_DOWN, !tiled ? launch_gemm_grouped(g, GEMM_MX_M16_N64, (int)W.max_tiles, st)
                                    : astat_supported(g) ? launch_astat(g, (int)W.max_tiles, st)
                                                         : launch_tiled(g, true, (int)W.max_tiles, st));
    }
    // zc = bf16(sum_j w_j y_j) in slot order: into the first Lt columns of [zc | h_s], or the output
    MOE_LAUNCH(MOE_KERNEL_COMBINE, launch_combine(Yb, Lt, r->inv, r->topk_w, T, K, lat ? Acat : static_cast<uint16_t *>(out),
                           lat ? ldcat : Lt, st));
    if (shared_apart(c) && hipStreamWaitEvent(st, h->join, 0) != hipSuccess)   // h_s from the second stream
        return MOE_ERR_HIP;
    if (lat && T <= SKINNY_MAX_M) {   // out = bf16([zc | h_s] [W_up | Wd_s]^T) from split-K partials
        float *partials = reinterpret_cast<float *>(ws + W.partials);
        const int64_t pstride = (int64_t)(H / 16) * SKINNY_TILE_FLOATS;
        SkinnyArgs g{Acat, ldcat, T, h->packed + h->off_outside, H, ldcat, partials, pstride};
        MOE_LAUNCH(MOE_KERNEL_OUT, launch_skinny_persist(g, 8, OUT_GROUPS, SKINNY_XSTEPS, st));
        MOE_LAUNCH(MOE_KERNEL_OUT_EPI, launch_out_epilogue(partials, pstride, skinny_splits(ldcat, SKINNY_XSTEPS), T, H,
                                                           static_cast<uint16_t *>(out), st));
    } else if (lat) {
        GemmArgs g{};
        g.A = Acat;
        g.lda = ldcat;
        g.B = h->packed + h->off_outside;
        g.M = T;
        g.N = H;
        g.K = ldcat;
        g.split = INT_MAX;
        g.lo = OutDesc{OUT_BF16, out, H, 0, H, nullptr};
        MOE_LAUNCH(MOE_KERNEL_OUT, (ring_preferred(g) ? launch_ring(g, st) : launch_tiled(g, false, 0, st)));
    }
    return MOE_OK;
}

moe_status check_route_args(moe_handle *h, const void *x, int32_t T, const float *logit_bias, const float *logits_in,
                            const float *logits_out, const moe_routing *r)
{
    if (!h || T < 0 || !r || !call_fits(&h->cfg, T))
        return MOE_ERR_INVALID_ARG;
    if (T == 0)
        return MOE_OK;
    if (logits_in ? (x || logit_bias || logits_out) : !x)
        return MOE_ERR_INVALID_ARG;
    if (!r->topk_ids || !r->topk_w || !r->counts || !r->offsets || !r->sorted_pairs || !r->inv)
        return MOE_ERR_INVALID_ARG;
    if (x && !aligned(x, 16))
        return MOE_ERR_INVALID_ARG;
    return MOE_OK;
}

moe_status check_forward_args(moe_handle *h, const void *x, int32_t T, const moe_routing *r, const void *out)
{
    if (!h || T < 0 || !r || !call_fits(&h->cfg, T))
        return MOE_ERR_INVALID_ARG;
    if (T == 0)
        return MOE_OK;
    if (!x || !out || !aligned(x, 16) || !aligned(out, 16) || x == out)
        return MOE_ERR_INVALID_ARG;
    if (!r->topk_w || !r->offsets || !r->sorted_pairs || !r->inv)
        return MOE_ERR_INVALID_ARG;
    return MOE_OK;
}

moe_status check_workspace(const WsLayout &W, const void *workspace, size_t workspace_bytes)
{
    if (!workspace || !aligned(workspace, ALIGN))
        return MOE_ERR_INVALID_ARG;
    if (workspace_bytes < (size_t)W.total)
        return MOE_ERR_BUFFER_TOO_SMALL;
    return MOE_OK;
}

} // namespace

extern "C" {

moe_status moe_route(moe_handle *h, const void *x, int32_t T, const float *logit_bias, const float *logits_in,
                     float *logits_out, const moe_routing *r, void *workspace, size_t workspace_bytes, void *stream)
{
    moe_status e = check_route_args(h, x, T, logit_bias, logits_in, logits_out, r);
    if (e != MOE_OK || T == 0)
        return e;
    const WsLayout W = ws_layout(&h->cfg, T);
    if ((e = check_workspace(W, workspace, workspace_bytes)) != MOE_OK)
        return e;
    uint8_t *ws = static_cast<uint8_t *>(workspace);
    hipStream_t st = static_cast<hipStream_t>(stream);
    TopkArgs ta;
    if ((e = router_impl(h, x, T, logit_bias, logits_in, logits_out, r, W, ws, st, ta)) != MOE_OK)
        return e;
    return select_impl(h, T, ta, r, W, ws, st, false);
}

moe_status moe_forward(moe_handle *h, const void *x, int32_t T, const moe_routing *r, void *out, void *workspace,
                       size_t workspace_bytes, void *stream)
{
    moe_status e = check_forward_args(h, x, T, r, out);
    if (e != MOE_OK || T == 0)
        return e;
    const WsLayout W = ws_layout(&h->cfg, T);
    if ((e = check_workspace(W, workspace, workspace_bytes)) != MOE_OK)
        return e;
    uint8_t *ws = static_cast<uint8_t *>(workspace);
    hipStream_t st = static_cast<hipStream_t>(stream);
    if ((e = xside_impl(h, x, T, r, W, ws, st, true)) != MOE_OK)
        return e;
    return experts_impl(h, x, T, r, out, W, ws, st);
}

} // extern "C"

namespace {

moe_status check_route_forward_args(moe_handle *h, const void *x, int32_t T, const float *logit_bias,
                                    const float *logits_out, const moe_routing *r, const void *out)
{
    moe_status e = check_route_args(h, x, T, logit_bias, nullptr, logits_out, r);
    if (e == MOE_OK)
        e = check_forward_args(h, x, T, r, out);
    if (e != MOE_OK || T == 0)
        return e;
    if ((const void *)logits_out == out || (const void *)logits_out == x)
        return MOE_ERR_INVALID_ARG;
    return MOE_OK;
}

// The launch sequence of moe_route_forward on workspace `ws` (layout W); arguments checked.
moe_status route_forward_impl(moe_handle *h, const void *x, int32_t T, const float *logit_bias, float *logits_out,
                              const moe_routing *r, void *out, const WsLayout &W, uint8_t *ws, hipStream_t st)
{
    moe_status e;
    if (h->cfg.has_latent_proj)
        e = front_impl(h, x, T, logit_bias, logits_out, r, W, ws, st);
    else {   // no x-side products: router, then the grouping builds the tile lists
        TopkArgs ta;
        e = router_impl(h, x, T, logit_bias, nullptr, logits_out, r, W, ws, st, ta);
        if (e == MOE_OK)
            e = select_impl(h, T, ta, r, W, ws, st, true);
    }
    if (e != MOE_OK)
        return e;
    return experts_impl(h, x, T, r, out, W, ws, st);
}

} // namespace

extern "C" {

moe_status moe_route_forward(moe_handle *h, const void *x, int32_t T, const float *logit_bias, float *logits_out,
                             const moe_routing *r, void *out, void *workspace, size_t workspace_bytes, void *stream)
{
    moe_status e = check_route_forward_args(h, x, T, logit_bias, logits_out, r, out);
    if (e != MOE_OK || T == 0)
        return e;
    const WsLayout W = ws_layout(&h->cfg, T);
    if ((e = check_workspace(W, workspace, workspace_bytes)) != MOE_OK)
        return e;
    return route_forward_impl(h, x, T, logit_bias, logits_out, r, out, W, static_cast<uint8_t *>(workspace),
                              static_cast<hipStream_t>(stream));
}

moe_status moe_route_forward_static(moe_handle *h, const void *x, int32_t T, const float *logit_bias,
                                    float *logits_out, const moe_routing *r, void *out, void *stream)
{
    moe_status e = check_route_forward_args(h, x, T, logit_bias, logits_out, r, out);
    if (e != MOE_OK || T == 0)
        return e;
    const WsLayout W = ws_layout(&h->cfg, T);
    if ((uint64_t)W.total > (uint64_t)MOE_STATIC_SCRATCH_BYTES)
        return MOE_ERR_BUFFER_TOO_SMALL;
    void *ws = nullptr;
    if ((e = scratch_address(&ws)) != MOE_OK)
        return e;
    // nothing in the workspace has to start at zero: every region a launch reads is written
    // earlier in the same call
    return route_forward_impl(h, x, T, logit_bias, logits_out, r, out, W, static_cast<uint8_t *>(ws),
                              static_cast<hipStream_t>(stream));
}

struct moe_graph {
    hipGraphExec_t exec;
};

moe_status moe_graph_create(moe_handle *h, const void *x, int32_t T, const float *logit_bias, float *logits_out,
                            const moe_routing *r, void *out, void *workspace, size_t workspace_bytes, moe_graph **g)
{
    if (!g)
        return MOE_ERR_INVALID_ARG;
    *g = nullptr;
    moe_status e = check_route_forward_args(h, x, T, logit_bias, logits_out, r, out);
    if (e != MOE_OK)
        return e;
    if (T == 0 || h->prof)
        return MOE_ERR_INVALID_ARG;
    const WsLayout W = ws_layout(&h->cfg, T);
    if ((e = check_workspace(W, workspace, workspace_bytes)) != MOE_OK)
        return e;
    hipStream_t cs = nullptr;
    if (hipStreamCreateWithFlags(&cs, hipStreamNonBlocking) != hipSuccess)
        return MOE_ERR_HIP;
    hipGraph_t graph = nullptr;
    hipGraphExec_t exec = nullptr;
    if (hipStreamBeginCapture(cs, hipStreamCaptureModeThreadLocal) != hipSuccess) {
        (void)hipStreamDestroy(cs);
        return MOE_ERR_HIP;
    }
    e = route_forward_impl(h, x, T, logit_bias, logits_out, r, out, W, static_cast<uint8_t *>(workspace), cs);
    const hipError_t ce = hipStreamEndCapture(cs, &graph);   // ends the capture whatever happened
    if (e == MOE_OK && (ce != hipSuccess || !graph))
        e = MOE_ERR_HIP;
    if (e == MOE_OK && hipGraphInstantiate(&exec, graph, nullptr, nullptr, 0) != hipSuccess)
        e = MOE_ERR_HIP;
    if (graph)
        (void)hipGraphDestroy(graph);
    (void)hipStreamDestroy(cs);
    if (e != MOE_OK)
        return e;
    moe_graph *gr = new (std::nothrow) moe_graph{exec};
    if (!gr) {
        (void)hipGraphExecDestroy(exec);
        return MOE_ERR_HIP;
    }
    *g = gr;
    return MOE_OK;
}

moe_status moe_graph_launch(moe_graph *g, void *stream)
{
    if (!g)
        return MOE_ERR_INVALID_ARG;
    return hip_status(hipGraphLaunch(g->exec, static_cast<hipStream_t>(stream)));
}

void moe_graph_destroy(moe_graph *g)
{
    if (!g)
        return;
    (void)hipGraphExecDestroy(g->exec);
    delete g;
}

moe_status moe_unpack_expert(moe_handle *h, int32_t e, int32_t which, void *out, void *stream)
{
    if (!h || !out || e < 0 || e >= h->cfg.n_experts || which < 0 || which > 2 || !aligned(out, 16))
        return MOE_ERR_INVALID_ARG;
    const moe_config *c = &h->cfg;
    hipStream_t st = static_cast<hipStream_t>(stream);
    uint16_t *o = static_cast<uint16_t *>(out);
    if (which < 2)
        return hip_status(launch_unpack_mx(h->packed + h->off_gateup + e * h->gateup_stride, 2 * (int64_t)c->inter,
                                           c->latent, 1, which, o, st));
    return hip_status(
        launch_unpack_mx(h->packed + h->off_down + e * h->down_stride, c->latent, c->inter, 0, 0, o, st));
}

} // extern "C"
