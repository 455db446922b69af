// Host runtime of the C ABI in include/moe.h: validation, buffer plans,
// workspace carving and kernel launches.  No allocation, no host sync (except
// moe_read_device_status).
#include <string.h>

#include <vector>

#include "../../include/moe.h"
#include "common.hpp"
#include "kernels.hpp"

using namespace moe;

namespace {

constexpr int kNumCUs = 256;      // MI355X compute units
constexpr int kBalanceRows = 320;  // bf16 machine balance: ~2.5 PFLOP/s over 8 TB/s, in rows
constexpr size_t kAlign = 256;

size_t align_up(size_t v) { return (v + kAlign - 1) & ~(kAlign - 1); }

struct Plan {
    int T, H, I, E, k, Et, Mb, nmb, slots, comm_cus, prec;
    bool shared, identity;
    int ld_tok_prow;  // k (+1 with the shared expert)
    int64_t rpad;     // padded GEMM rows of one minibatch
    int max_mtiles;
    // packed weights (bytes)
    size_t pk_w1t, pk_w2t, packed;
    // forward workspace (bytes)
    size_t ws_status, ws_idx, ws_w, ws_slot0, slot_bytes, ws_fwd;
    size_t sl_hdr, sl_mt, sl_prow_token, sl_tok_prow, sl_h, sl_y;
    // saved (bytes)
    size_t sv_idx, sv_w, saved;
    size_t ws_bwd;
};

moe_status validate(const moe_cfg* c) {
    if (!c) return MOE_E_INVALID;
    if (c->T < 1 || c->E < 1 || c->k < 1 || c->k > c->E || c->H < 1 || c->I < 1) return MOE_E_INVALID;
    if (c->minibatch < 0 || c->ring_slots < 0 || c->comm_cus < 0) return MOE_E_INVALID;
    if (c->prec != MOE_PREC_BF16 && c->prec != MOE_PREC_MXFP8) return MOE_E_INVALID;
    if (c->flags & ~(uint32_t)(MOE_F_SHARED_EXPERT | MOE_F_IDENTITY_EXPERTS)) return MOE_E_INVALID;
    if (c->H % 64 || c->I % 64 || c->E > kMaxExperts || c->k > kMaxTopK) return MOE_E_UNSUPPORTED;
    if ((int64_t)c->T * c->k > (1ll << 30) || (int64_t)c->T * c->H > (1ll << 40)) return MOE_E_UNSUPPORTED;
    return MOE_OK;
}

int auto_minibatch(const moe_cfg* c) {
    // Smallest multiple of 256 tokens such that (i) the gate/up GEMM has at least
    // two full waves of output tiles on the GEMM CUs and (ii) the mean rows per
    // expert reach the machine balance, so weights are not re-streamed for a
    // handful of rows.  Then spread T evenly over that many minibatches.
    const int nt1 = ceil_div(2 * c->I, BN);
    int mb = c->T;
    for (int m = 256; m < c->T; m += 256) {
        const int64_t tiles = (int64_t)ceil_div(m * c->k, BM) * nt1;
        if (tiles >= 2 * kNumCUs && (int64_t)m * c->k >= (int64_t)kBalanceRows * c->E) {
            mb = m;
            break;
        }
    }
    const int nmb = c->T / mb > 0 ? c->T / mb : 1;
    mb = ceil_div(ceil_div(c->T, nmb), 64) * 64;
    return mb < c->T ? mb : c->T;
}

moe_status make_plan(const moe_cfg* c, Plan* p) {
    moe_status st = validate(c);
    if (st != MOE_OK) return st;
    memset(p, 0, sizeof(*p));
    p->T = c->T; p->H = c->H; p->I = c->I; p->E = c->E; p->k = c->k; p->prec = c->prec;
    p->shared = (c->flags & MOE_F_SHARED_EXPERT) != 0;
    p->identity = (c->flags & MOE_F_IDENTITY_EXPERTS) != 0;
    if (p->prec != MOE_PREC_BF16) return MOE_E_UNSUPPORTED;
    p->Et = c->E + (p->shared ? 1 : 0);
    p->Mb = c->minibatch > 0 ? (c->minibatch < c->T ? c->minibatch : c->T) : auto_minibatch(c);
    p->nmb = ceil_div(c->T, p->Mb);
    p->slots = c->ring_slots > 0 ? c->ring_slots : 2;
    if (p->slots > p->nmb) p->slots = p->nmb;
    p->comm_cus = c->comm_cus;
    p->ld_tok_prow = c->k + (p->shared ? 1 : 0);
    const int64_t rows = (int64_t)p->Mb * p->ld_tok_prow;
    // sum over experts of ceil(c_e / BM) <= ceil(rows / BM) + Et - 1
    p->max_mtiles = (int)(ceil_div((int)rows, BM) + p->Et - 1);
    p->rpad = (int64_t)p->max_mtiles * BM;

    const size_t H = c->H, I = c->I, Et = p->Et;
    p->pk_w1t = 0;
    p->pk_w2t = align_up(p->pk_w1t + Et * 2 * I * H * 2);
    p->packed = align_up(p->pk_w2t + Et * H * I * 2);

    const size_t Tk = (size_t)c->T * c->k;
    p->ws_status = 0;
    p->ws_idx = kAlign;
    p->ws_w = align_up(p->ws_idx + Tk * 4);
    p->ws_slot0 = align_up(p->ws_w + Tk * 4);
    size_t o = 0;
    p->sl_hdr = o; o = align_up(o + sizeof(LayoutHeader));
    p->sl_mt = o; o = align_up(o + (Et + 1) * 4);
    p->sl_prow_token = o; o = align_up(o + (size_t)p->rpad * 4);
    p->sl_tok_prow = o; o = align_up(o + (size_t)p->Mb * p->ld_tok_prow * 4);
    p->sl_h = o; o = align_up(o + (size_t)p->rpad * I * 2);
    p->sl_y = o; o = align_up(o + (size_t)p->rpad * H * 2);
    p->slot_bytes = o;
    p->ws_fwd = p->ws_slot0 + (size_t)p->slots * p->slot_bytes;

    p->sv_idx = 0;
    p->sv_w = align_up(Tk * 4);
    p->saved = align_up(p->sv_w + Tk * 4);
    p->ws_bwd = kAlign;
    return MOE_OK;
}

bool aligned(const void* ptr, size_t a) { return ((uintptr_t)ptr & (a - 1)) == 0; }

// Optional per-launch event timing (moe_timing_enable / moe_timing_read).
struct Timing {
    bool on = false;
    std::vector<hipEvent_t> ev;  // 2 per launch
    std::vector<int> kind;
    int used = 0, dropped = 0;
};
Timing g_timing;
constexpr int kTimingPairs = 4096;

struct TimedLaunch {
    int slot = -1;
    hipStream_t s;
    TimedLaunch(moe_kernel_kind k, hipStream_t stream) : s(stream) {
        if (!g_timing.on) return;
        if (g_timing.used >= kTimingPairs) { ++g_timing.dropped; return; }
        slot = g_timing.used++;
        g_timing.kind[slot] = k;
        (void)hipEventRecord(g_timing.ev[2 * slot], s);
    }
    ~TimedLaunch() {
        if (slot >= 0) (void)hipEventRecord(g_timing.ev[2 * slot + 1], s);
    }
};

#define TIMED(kind, stream, call) \
    do {                          \
        TimedLaunch tl_(kind, stream); \
        call;                     \
    } while (0)

moe_status check_launch() { return hipGetLastError() == hipSuccess ? MOE_OK : MOE_E_HIP; }

}  // namespace

extern "C" {

const char* moe_status_string(moe_status s) {
    switch (s) {
        case MOE_OK: return "ok";
        case MOE_E_INVALID: return "invalid argument";
        case MOE_E_UNSUPPORTED: return "unsupported configuration";
        case MOE_E_WORKSPACE: return "buffer too small";
        case MOE_E_HIP: return "HIP runtime error";
        case MOE_E_DEVICE: return "device-side error";
    }
    return "unknown status";
}

int32_t moe_abi_version(void) { return MOE_ABI_VERSION; }

moe_status moe_validate_cfg(const moe_cfg* cfg) { return validate(cfg); }

moe_status moe_query_sizes(const moe_cfg* cfg, moe_sizes* out) {
    if (!out) return MOE_E_INVALID;
    Plan p;
    moe_status st = make_plan(cfg, &p);
    if (st != MOE_OK) return st;
    out->packed_weights = p.packed;
    out->workspace_fwd = p.ws_fwd;
    out->saved = p.saved;
    out->workspace_bwd = p.ws_bwd;
    out->minibatch = p.Mb;
    out->ring_slots = p.slots;
    out->num_minibatches = p.nmb;
    out->comm_cus = p.comm_cus;
    return MOE_OK;
}

moe_status moe_prepare_weights(const moe_cfg* cfg, const uint16_t* Wg, const uint16_t* Wu,
                               const uint16_t* Wd, const uint16_t* Wsg, const uint16_t* Wsu,
                               const uint16_t* Wsd, void* packed, size_t packed_bytes, void* stream) {
    Plan p;
    moe_status st = make_plan(cfg, &p);
    if (st != MOE_OK) return st;
    if (!Wg || !Wu || !Wd || !packed) return MOE_E_INVALID;
    if (p.shared && (!Wsg || !Wsu || !Wsd)) return MOE_E_INVALID;
    if (!aligned(packed, kAlign)) return MOE_E_INVALID;
    if (packed_bytes < p.packed) return MOE_E_WORKSPACE;
    hipStream_t s = (hipStream_t)stream;
    uint8_t* base = (uint8_t*)packed;
    uint16_t* W1t = (uint16_t*)(base + p.pk_w1t);
    uint16_t* W2t = (uint16_t*)(base + p.pk_w2t);
    const size_t H = p.H, I = p.I;
    launch_pack_gate_up(Wg, Wu, p.E, p.H, p.I, W1t, s);
    launch_transpose(Wd, p.E, p.I, p.H, W2t, s);
    if (p.shared) {
        launch_pack_gate_up(Wsg, Wsu, 1, p.H, p.I, W1t + (size_t)p.E * 2 * I * H, s);
        launch_transpose(Wsd, 1, p.I, p.H, W2t + (size_t)p.E * H * I, s);
    }
    return check_launch();
}

moe_status moe_route(const moe_cfg* cfg, const uint16_t* x, const float* Wr, const float* bias,
                     int32_t* topk_idx, float* topk_w, float* logits, void* stream) {
    moe_status st = validate(cfg);
    if (st != MOE_OK) return st;
    if (!x || !Wr || !topk_idx || !topk_w) return MOE_E_INVALID;
    TIMED(MOE_K_ROUTE, (hipStream_t)stream,
          launch_route(x, Wr, bias, cfg->T, cfg->H, cfg->E, cfg->k, topk_idx, topk_w, logits, (hipStream_t)stream));
    return check_launch();
}

moe_status moe_dispatch_layout(const moe_cfg* cfg, const int32_t* topk_idx, int32_t* counts,
                               int32_t* offsets, int32_t* row_token, int32_t* tok_row, void* stream) {
    moe_status st = validate(cfg);
    if (st != MOE_OK) return st;
    if (!topk_idx || !counts || !offsets || !row_token || !tok_row) return MOE_E_INVALID;
    LayoutOut o;
    memset(&o, 0, sizeof(o));
    o.counts = counts;
    o.offsets = offsets;
    o.row_token = row_token;
    o.tok_row = tok_row;
    TIMED(MOE_K_LAYOUT, (hipStream_t)stream, launch_layout(topk_idx, cfg->T, cfg->E, cfg->k, 0, o, (hipStream_t)stream));
    return check_launch();
}

moe_status moe_layer_fwd(const moe_cfg* cfg, const moe_weights* w, const uint16_t* x, uint16_t* out,
                         void* saved, size_t saved_bytes, void* ws, size_t ws_bytes, void* stream) {
    Plan p;
    moe_status st = make_plan(cfg, &p);
    if (st != MOE_OK) return st;
    if (!w || !w->Wr || !w->packed || !x || !out || !ws) return MOE_E_INVALID;
    if (!aligned(x, 16) || !aligned(out, 16) || !aligned(ws, kAlign) || !aligned(w->packed, kAlign))
        return MOE_E_INVALID;
    if (saved && !aligned(saved, kAlign)) return MOE_E_INVALID;
    if (w->packed_bytes < p.packed || ws_bytes < p.ws_fwd) return MOE_E_WORKSPACE;
    if (saved && saved_bytes < p.saved) return MOE_E_WORKSPACE;
    hipStream_t s = (hipStream_t)stream;
    uint8_t* wsb = (uint8_t*)ws;
    int32_t* idx = saved ? (int32_t*)((uint8_t*)saved + p.sv_idx) : (int32_t*)(wsb + p.ws_idx);
    float* gw = saved ? (float*)((uint8_t*)saved + p.sv_w) : (float*)(wsb + p.ws_w);
    const uint8_t* pk = (const uint8_t*)w->packed;
    const uint16_t* W1t = (const uint16_t*)(pk + p.pk_w1t);
    const uint16_t* W2t = (const uint16_t*)(pk + p.pk_w2t);

    TIMED(MOE_K_ROUTE, s, launch_route(x, w->Wr, w->bias, p.T, p.H, p.E, p.k, idx, gw, nullptr, s));
    const int grid = kNumCUs;
    for (int b = 0; b < p.nmb; ++b) {
        const int t0 = b * p.Mb;
        const int Tm = (p.T - t0) < p.Mb ? (p.T - t0) : p.Mb;
        uint8_t* slot = wsb + p.ws_slot0 + (size_t)(b % p.slots) * p.slot_bytes;
        LayoutHeader* hdr = (LayoutHeader*)(slot + p.sl_hdr);
        int32_t* mt = (int32_t*)(slot + p.sl_mt);
        int32_t* prow_token = (int32_t*)(slot + p.sl_prow_token);
        int32_t* tok_prow = (int32_t*)(slot + p.sl_tok_prow);
        uint16_t* hbuf = (uint16_t*)(slot + p.sl_h);
        uint16_t* ybuf = (uint16_t*)(slot + p.sl_y);

        LayoutOut o;
        memset(&o, 0, sizeof(o));
        o.hdr = hdr;
        o.mt_start = mt;
        o.prow_token = prow_token;
        o.tok_prow = tok_prow;
        o.tok_prow_ld = p.ld_tok_prow;
        o.token_base = t0;
        TIMED(MOE_K_LAYOUT, s, launch_layout(idx + (size_t)t0 * p.k, Tm, p.E, p.k, p.shared ? 1 : 0, o, s));

        if (p.identity) {
            TIMED(MOE_K_GATHER, s, launch_gather_rows(x, p.H, prow_token, hdr, (int)p.rpad, ybuf, p.H, s));
        } else {
            GemmArgs g1;
            g1.A = x; g1.a_row_map = prow_token; g1.lda = p.H;
            g1.B = W1t; g1.b_stride = (int64_t)2 * p.I * p.H;
            g1.C = hbuf; g1.ldc = p.I;
            g1.N = 2 * p.I; g1.K = p.H;
            g1.mt_start = mt; g1.hdr = hdr; g1.Et = p.Et;
            TIMED(MOE_K_GEMM_GATE_UP, s, launch_grouped_gemm(g1, kEpiSwiGLU, grid, s));
            GemmArgs g2;
            g2.A = hbuf; g2.a_row_map = nullptr; g2.lda = p.I;
            g2.B = W2t; g2.b_stride = (int64_t)p.H * p.I;
            g2.C = ybuf; g2.ldc = p.H;
            g2.N = p.H; g2.K = p.I;
            g2.mt_start = mt; g2.hdr = hdr; g2.Et = p.Et;
            TIMED(MOE_K_GEMM_DOWN, s, launch_grouped_gemm(g2, kEpiStore, grid, s));
        }
        TIMED(MOE_K_COMBINE, s,
              launch_combine(ybuf, p.H, tok_prow, p.ld_tok_prow, gw + (size_t)t0 * p.k, p.k,
                             (p.shared && !p.identity) ? 1 : 0, p.H, Tm, out + (size_t)t0 * p.H, s));
    }
    return check_launch();
}

moe_status moe_layer_bwd(const moe_cfg* cfg, const moe_weights* w, const uint16_t* x, const uint16_t* dout,
                         const void* saved, size_t saved_bytes, uint16_t* dx, float* dWg, float* dWu,
                         float* dWd, float* dWr, float* dWs, float* dgate, void* ws, size_t ws_bytes,
                         void* stream) {
    Plan p;
    moe_status st = make_plan(cfg, &p);
    if (st != MOE_OK) return st;
    (void)w; (void)x; (void)dout; (void)saved; (void)saved_bytes; (void)dx; (void)dWg; (void)dWu;
    (void)dWd; (void)dWr; (void)dWs; (void)dgate; (void)ws; (void)ws_bytes; (void)stream;
    return MOE_E_UNSUPPORTED;
}

moe_status moe_read_device_status(void* ws, void* stream, int32_t* code, int32_t* detail) {
    if (!ws || !code || !detail) return MOE_E_INVALID;
    if (hipStreamSynchronize((hipStream_t)stream) != hipSuccess) return MOE_E_HIP;
    int32_t h[2] = {0, 0};
    if (hipMemcpy(h, ws, sizeof(h), hipMemcpyDeviceToHost) != hipSuccess) return MOE_E_HIP;
    *code = h[0];
    *detail = h[1];
    if (h[0] != 0) {
        const int32_t z[2] = {0, 0};
        if (hipMemcpy(ws, z, sizeof(z), hipMemcpyHostToDevice) != hipSuccess) return MOE_E_HIP;
        return MOE_E_DEVICE;
    }
    return MOE_OK;
}

moe_status moe_timing_enable(int32_t on) {
    if (on) {
        if (g_timing.ev.empty()) {
            g_timing.ev.resize(2 * kTimingPairs);
            g_timing.kind.resize(kTimingPairs);
            for (auto& e : g_timing.ev)
                if (hipEventCreate(&e) != hipSuccess) {
                    g_timing.ev.clear();
                    return MOE_E_HIP;
                }
        }
        g_timing.used = 0;
        g_timing.dropped = 0;
    }
    g_timing.on = on != 0;
    return MOE_OK;
}

moe_status moe_timing_read(moe_kernel_times* out) {
    if (!out) return MOE_E_INVALID;
    memset(out, 0, sizeof(*out));
    for (int i = 0; i < g_timing.used; ++i) {
        if (hipEventSynchronize(g_timing.ev[2 * i + 1]) != hipSuccess) return MOE_E_HIP;
        float ms = 0.0f;
        if (hipEventElapsedTime(&ms, g_timing.ev[2 * i], g_timing.ev[2 * i + 1]) != hipSuccess) return MOE_E_HIP;
        out->launches[g_timing.kind[i]] += 1;
        out->ms[g_timing.kind[i]] += ms;
    }
    out->dropped = g_timing.dropped;
    return MOE_OK;
}

}  // extern "C"
