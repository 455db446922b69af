// Host runtime of the C ABI in include/moe.h: validation, buffer plans,
// workspace carving and kernel launches.  No allocation, no host sync (except
// moe_read_device_status).
#include <string.h>

#include <algorithm>
#include <mutex>
#include <vector>

#include "../../include/moe.h"
#include "common.hpp"
#include "kernels.hpp"

using namespace moe;

namespace {

constexpr int kNumCUs = 256;      // MI355X compute units
constexpr int kBalanceRows = 320;  // bf16 machine balance: ~2.5 PFLOP/s over 8 TB/s, in rows
constexpr int kPadShare = 32;      // automatic minibatch: expected padding rows at most 1/32 of the rows
constexpr int kGroupTokens = 8192; // layer kernel: tokens per GEMM phase (minibatches grouped up to this)
constexpr int kBwdChunkTokens = 5120;  // backward: tokens per phase chunk (minibatches grouped up to this)
constexpr int kBwdChunkTokensShared = 20480;  // the same with the shared expert
constexpr int kMaxGroup = 4;
constexpr uint64_t kSpinTicks = 200000000;  // 2 s at the 100 MHz s_memrealtime clock: bound of every device wait
constexpr size_t kAlign = 256;

size_t align_up(size_t v) { return (v + kAlign - 1) & ~(kAlign - 1); }

struct Plan {
    int T, H, I, E, k, Et, Mb, nmb, slots, comm_cus, prec;
    int group;  // minibatches per phase of the layer kernel
    int bchunk; // minibatches per phase chunk of the backward
    bool shared, identity;
    int ld_tok_prow;  // k (+1 with the shared expert)
    int64_t rpad;     // padded GEMM rows of one minibatch
    int max_mtiles;
    // packed weights (bytes): forward gate|up [Et][2I][H], down [Et][H][I];
    // backward down [Et][I][H] and gate|up rows [Et][H][2I]
    size_t pk_w1t, pk_w2t, pk_wd, pk_wgu, packed;
    // MXFP8 copies of the routed experts' weights: codes and scales, forward
    // (along H for gate|up, along I for down) and input-gradient (Wd along H,
    // Wg|Wu along I)
    size_t pk_w1q, pk_s1, pk_w2q, pk_s2, pk_wdq, pk_sd, pk_wguq, pk_sgu;
    bool mx;
    // forward workspace (bytes): routing, MXFP8 x, every minibatch's layout
    // (first-tile maps [nmb][Et+1], then nmb blocks of lay_bytes), layer-kernel
    // counters, ring slots (h, Y, MXFP8 h codes and scales)
    size_t ws_status, ws_idx, ws_w, ws_mt, ws_prs, ws_rows, ws_lay0, ws_cnt, ws_slot0, slot_bytes, ws_fwd;
    size_t sl_h, sl_y, sl_hq, sl_sh;
    bool mega;  // forward through the persistent layer kernel
    size_t ws_xq, ws_sx;  // MXFP8 codes and scales of x
    // saved (bytes): routing, then per minibatch g|u [rpad][2I] (bf16, or fp32
    // under MXFP8) and Y [rpad][H]
    size_t sv_idx, sv_w, sv_mb0, sv_mb, sv_y, sv_hs, saved;
    // backward workspace (bytes)
    size_t wb_wrt, wb_mt, wb_prs, wb_rows, wb_lay0, lay_bytes, ly_hdr, ly_prow_token, ly_tok_prow, ly_prow_slot;
    size_t wb_dgu, wb_hw, wb_dsel, wb_dh, wb_dx, wb_dgp, wb_roww, ws_bwd;
    size_t wb_dyq, wb_sdy, wb_dguq, wb_sdgu;  // MXFP8 operands of the input-gradient GEMMs
    bool mxw;  // MXFP8 weight gradients of the routed experts
    // their operands, one copy per minibatch: codes and scales of dY, x, dG | dU, h
    size_t wb_dytq, wb_sdyt, wb_xgtq, wb_sxgt, wb_dgutq, wb_sdgut, wb_htq, wb_sht;
    size_t wb_dlog, wb_dwrp;                  // dense d out / d logits, router-gradient partial sums
};

moe_status validate(const moe_cfg* c) {
    if (!c) return MOE_E_INVALID;
    if (c->T < 1 || c->E < 1 || c->k < 1 || c->k > c->E || c->H < 1 || c->I < 1) return MOE_E_INVALID;
    if (c->minibatch < 0 || c->ring_slots < 0 || c->comm_cus < 0) return MOE_E_INVALID;
    if (c->prec != MOE_PREC_BF16 && c->prec != MOE_PREC_MXFP8) return MOE_E_INVALID;
    if (c->flags & ~(uint32_t)(MOE_F_SHARED_EXPERT | MOE_F_IDENTITY_EXPERTS | MOE_F_LAUNCH_PER_GEMM |
                               MOE_F_DEBUG_DROP_SIGNAL | MOE_F_BF16_WGRAD))
        return MOE_E_INVALID;
    if ((c->flags & MOE_F_BF16_WGRAD) && c->prec != MOE_PREC_MXFP8) return MOE_E_INVALID;
    if (c->H % 64 || c->I % 64 || c->E > kMaxExperts || c->k > kMaxTopK) return MOE_E_UNSUPPORTED;
    if ((int64_t)c->T * c->k > (1ll << 30) || (int64_t)c->T * c->H > (1ll << 40)) return MOE_E_UNSUPPORTED;
    return MOE_OK;
}

int auto_minibatch(const moe_cfg* c) {
    // Smallest multiple of 256 tokens such that (i) the gate/up GEMM has at least
    // two full waves of output tiles on the GEMM CUs, (ii) the mean rows per
    // expert reach the machine balance, so weights are not re-streamed for a
    // handful of rows, and (iii) the padding of the experts' padded rows
    // (kSegRows/2 rows per expert expected) is at most 1/kPadShare of the
    // minibatch's rows.  Measured (layer kernel, 16384 tokens, one box): at
    // H=7168, I=2048, E=32, k=8 bf16 14.21 / 12.24 / 12.18 / 11.13 / 11.11 /
    // 10.67 ms and MXFP8 (Zipf router) 8.40 / 7.45 / 7.40 / 6.66 / 6.49 /
    // 6.35 ms at minibatches of 1024 / 2048 / 2560 / 4096 / 6144 / 8192, and
    // the rule picks 8192; at H=2048, I=1024, E=64, k=6 with 4096 tokens,
    // 1.505 / 0.806 / 0.509 / 0.491 ms at 512 / 1024 / 2048 / 4096, and the
    // rule picks one minibatch of 4096.  Then spread T evenly over that many
    // minibatches.
    const int nt1 = ceil_div(2 * c->I, BN);
    int mb = c->T;
    for (int m = 256; m < c->T; m += 256) {
        const int64_t tiles = (int64_t)ceil_div(m * c->k, BM) * nt1;
        const int64_t rows = (int64_t)m * c->k;
        if (tiles >= 2 * kNumCUs && rows >= (int64_t)kBalanceRows * c->E &&
            rows >= (int64_t)kPadShare * c->E * (kSegRows / 2)) {
            mb = m;
            break;
        }
    }
    const int nmb = c->T / mb > 0 ? c->T / mb : 1;
    mb = ceil_div(ceil_div(c->T, nmb), 64) * 64;
    return mb < c->T ? mb : c->T;
}

// Workgroups the layer kernel dedicates to combine when the cfg leaves it to
// the library.  Dedicated workgroups take their CUs' share of the GEMM
// throughput, and on one GPU no GEMM phase leaves CUs idle for them to use:
// every active expert has at least one M tile per N tile, so even a few
// dozen tokens give more gate|up tiles than CUs.  Combine therefore runs as
// tiles of the GEMM workgroups (0).  Measured (layer kernel, one box):
// H=7168, I=2048, E=32, k=8, 16384 tokens in minibatches of 2560: bf16
// 12.18 ms with combine tiles against 17.55 / 14.14 / 13.44 ms with 8 / 16 /
// 32 combine workgroups, MXFP8 7.47 against 13.17 / 9.58 / 8.53 ms;
// H=2048, I=1024, E=64, k=6, 4096 tokens: combine tiles fastest at every
// minibatch of 512 / 1024 / 2048 / 4096 (e.g. 0.491 against 1.280 / 0.906 ms
// with 8 / 16 at 4096).  With several GPUs the communication role would also
// drive link transfers; that is out of this build's scope.
int auto_comm_cus(const moe_cfg*) { return 0; }

moe_status make_plan(const moe_cfg* c, Plan* p) {
    moe_status st = validate(c);
    if (st != MOE_OK) return st;
    memset(p, 0, sizeof(*p));
    p->T = c->T; p->H = c->H; p->I = c->I; p->E = c->E; p->k = c->k; p->prec = c->prec;
    p->shared = (c->flags & MOE_F_SHARED_EXPERT) != 0;
    p->identity = (c->flags & MOE_F_IDENTITY_EXPERTS) != 0;
    p->mx = p->prec == MOE_PREC_MXFP8;
    p->mxw = p->mx && !(c->flags & MOE_F_BF16_WGRAD);
    p->Et = c->E + (p->shared ? 1 : 0);
    p->Mb = c->minibatch > 0 ? (c->minibatch < c->T ? c->minibatch : c->T) : auto_minibatch(c);
    p->nmb = ceil_div(c->T, p->Mb);
    // The layer kernel runs its GEMM phases over groups of minibatches of about
    // kGroupTokens tokens (an expert's weight panels then serve that many
    // tokens' rows), with three groups of ring slots in flight.
    const int g_auto = std::max(1, std::min({kMaxGroup, kGroupTokens / p->Mb, p->nmb}));
    // The backward runs its phases over chunks of minibatches of about
    // kBwdChunkTokens tokens; with the shared expert, whose GEMMs have only
    // a minibatch's tokens each, of up to kBwdChunkTokensShared (every
    // minibatch at once for 16384 tokens in minibatches of 2560).
    const int chunk_tokens = (c->flags & MOE_F_SHARED_EXPERT) ? kBwdChunkTokensShared : kBwdChunkTokens;
    p->bchunk = std::max(1, std::min(chunk_tokens / p->Mb, p->nmb));
    p->group = c->ring_slots > 0 ? std::max(1, std::min(c->ring_slots / 3, g_auto)) : g_auto;
    p->slots = c->ring_slots > 0 ? c->ring_slots : 3 * p->group;
    p->slots = std::min(p->slots, ceil_div(p->nmb, p->group) * p->group);  // no slot without a minibatch
    p->slots -= p->slots % p->group;
    p->comm_cus = c->comm_cus > 0 ? c->comm_cus : auto_comm_cus(c);  // dedicated combine workgroups
    // The layer kernel's tile sequence runs gate|up(b+1) before down(b), so a
    // ring of one slot would make gate|up(b+1) wait on a later tile.  Identity
    // experts take the per-GEMM path.
    p->mega = !(c->flags & MOE_F_LAUNCH_PER_GEMM) && !p->identity && p->comm_cus < kNumCUs - 8;
    p->ld_tok_prow = c->k + (p->shared ? 1 : 0);
    const int64_t rows = (int64_t)p->Mb * p->ld_tok_prow;
    // sum over experts of ceil(c_e / BM) <= ceil(rows / BM) + Et - 1
    p->max_mtiles = (int)(ceil_div((int)rows, BM) + p->Et - 1);
    p->rpad = (int64_t)p->max_mtiles * BM;
    // The GEMM tiles address a row of an operand by a 32-bit byte offset from
    // the operand's (64-bit) base: the token matrix [T][H] and dout (gathered
    // rows), a minibatch's padded-row matrices ([rpad][H], [rpad][2I] and their
    // transposes) and one expert's weights ([2I][H]), bf16.
    {
        const int64_t lim = 1ll << 32, rp = p->rpad;
        if ((int64_t)c->T * c->H * 2 >= lim || rp * c->H * 2 >= lim || rp * 2 * c->I * 2 >= lim ||
            (int64_t)2 * c->I * c->H * 2 >= lim)
            return MOE_E_UNSUPPORTED;
    }

    const size_t H = c->H, I = c->I, Et = p->Et;
    p->pk_w1t = 0;
    p->pk_w2t = align_up(p->pk_w1t + Et * 2 * I * H * 2);
    p->pk_wd = align_up(p->pk_w2t + Et * H * I * 2);
    p->pk_wgu = align_up(p->pk_wd + Et * I * H * 2);
    size_t o = align_up(p->pk_wgu + Et * H * 2 * I * 2);
    if (p->mx) {
        const size_t E = c->E;
        p->pk_w1q = o; o = align_up(o + E * 2 * I * H);
        p->pk_s1 = o; o = align_up(o + E * mx_groups(H) * 2 * I * 4);
        p->pk_w2q = o; o = align_up(o + E * H * I);
        p->pk_s2 = o; o = align_up(o + E * mx_groups(I) * H * 4);
        p->pk_wdq = o; o = align_up(o + E * I * H);
        p->pk_sd = o; o = align_up(o + E * mx_groups(H) * I * 4);
        p->pk_wguq = o; o = align_up(o + E * H * 2 * I);
        p->pk_sgu = o; o = align_up(o + E * mx_groups(2 * I) * H * 4);
    }
    p->packed = o;

    const size_t Tk = (size_t)c->T * c->k;
    p->ws_status = 0;
    p->ws_idx = kAlign;
    p->ws_w = align_up(p->ws_idx + Tk * 4);
    o = align_up(p->ws_w + Tk * 4);
    if (p->mx) {
        p->ws_xq = o; o = align_up(o + (size_t)c->T * H);
        p->ws_sx = o; o = align_up(o + (size_t)mx_groups(H) * c->T * 4);
    }
    {  // one minibatch's layout block (also used by the backward)
        size_t l = 0;
        p->ly_hdr = l; l = align_up(l + sizeof(LayoutHeader));
        p->ly_prow_token = l; l = align_up(l + (size_t)p->rpad * 4);
        p->ly_tok_prow = l; l = align_up(l + (size_t)p->Mb * p->ld_tok_prow * 4);
        p->ly_prow_slot = l; l = align_up(l + (size_t)p->rpad * 4);
        p->lay_bytes = l;
    }
    p->ws_mt = o; o = align_up(o + (size_t)p->nmb * (Et + 1) * 4);
    p->ws_prs = o; o = align_up(o + (size_t)p->nmb * (Et + 1) * 4);
    p->ws_rows = o; o = align_up(o + (size_t)p->nmb * (Et + 1) * 4);
    p->ws_lay0 = o; o = align_up(o + (size_t)p->nmb * p->lay_bytes);
    p->ws_cnt = o; o = align_up(o + (size_t)(3 * p->nmb + 1) * 4);
    p->ws_slot0 = o;
    o = 0;
    p->sl_h = o; o = align_up(o + (size_t)p->rpad * I * 2);
    p->sl_y = o; o = align_up(o + (size_t)p->rpad * H * 2);
    if (p->mx) {
        p->sl_hq = o; o = align_up(o + (size_t)p->rpad * I);
        p->sl_sh = o; o = align_up(o + (size_t)mx_groups(I) * p->rpad * 4);
    }
    p->slot_bytes = o;
    p->ws_fwd = p->ws_slot0 + (size_t)p->slots * p->slot_bytes;

    const size_t rp = (size_t)p->rpad, nmb = (size_t)p->nmb;
    p->sv_idx = 0;
    p->sv_w = align_up(Tk * 4);
    p->sv_mb0 = align_up(p->sv_w + Tk * 4);
    p->sv_y = align_up(rp * 2 * I * (p->mx ? 4 : 2));  // g|u: fp32 under MXFP8 (its quantisation input)
    p->sv_mb = align_up(p->sv_y + rp * H * 2);
    // MXFP8 with the shared expert: its bf16 h rows, written by the shared
    // expert's own forward launches before the layer kernel
    p->sv_hs = p->sv_mb;
    if (p->mx && p->shared) p->sv_mb = align_up(p->sv_hs + rp * I * 2);
    p->saved = p->sv_mb0 + nmb * p->sv_mb;

    o = kAlign;  // device status word
    p->wb_wrt = o; o = align_up(o + (size_t)c->E * H * 4);
    p->wb_mt = o; o = align_up(o + nmb * (Et + 1) * 4);
    p->wb_prs = o; o = align_up(o + nmb * (Et + 1) * 4);
    p->wb_rows = o; o = align_up(o + nmb * (Et + 1) * 4);
    p->wb_lay0 = o; o += nmb * p->lay_bytes;
    // bf16 weight-gradient row operands of every minibatch (the other
    // operands, x and dout, are read through the row map): dG | dU, which the
    // bf16 gate|up input-gradient GEMM also reads, and w * h
    p->wb_dgu = o; o = align_up(o + nmb * rp * 2 * I * 2);
    p->wb_hw = o; o = align_up(o + nmb * rp * I * 2);
    p->wb_dsel = o; o = align_up(o + nmb * rp * 4);
    // one copy per minibatch of a backward chunk: the chunk's input-gradient
    // GEMMs run as one launch over its minibatches
    const size_t nc = (size_t)p->bchunk;
    // no row-major dY: the bf16 down input-gradient GEMM gathers dout rows and
    // scales each output row by its weight (row_w); the MXFP8 one reads the
    // quantised dY
    p->wb_roww = o; o = align_up(o + nc * rp * 4);
    p->wb_dh = o; o = align_up(o + nc * rp * I * (p->mx ? 4 : 2));
    p->wb_dx = o; o = align_up(o + nc * rp * H * 2);
    p->wb_dgp = o; o = align_up(o + nc * rp * (H / 64) * 4);
    p->wb_dlog = o; o = align_up(o + (size_t)c->T * c->E * 4);
    p->wb_dwrp = o; o = align_up(o + (size_t)dwr_chunks(c->T) * H * c->E * 4);
    if (p->mx) {
        p->wb_dyq = o; o = align_up(o + nc * rp * H);
        p->wb_sdy = o; o = align_up(o + nc * mx_groups(H) * rp * 4);
        p->wb_dguq = o; o = align_up(o + nc * rp * 2 * I);
        p->wb_sdgu = o; o = align_up(o + nc * mx_groups(2 * I) * rp * 4);
    }
    if (p->mxw) {  // rpad is a multiple of 256: whole scale groups of 128 rows
        p->wb_dytq = o; o = align_up(o + nmb * H * rp);
        p->wb_sdyt = o; o = align_up(o + nmb * mx_groups(rp) * H * 4);
        p->wb_xgtq = o; o = align_up(o + nmb * H * rp);
        p->wb_sxgt = o; o = align_up(o + nmb * mx_groups(rp) * H * 4);
        p->wb_dgutq = o; o = align_up(o + nmb * 2 * I * rp);
        p->wb_sdgut = o; o = align_up(o + nmb * mx_groups(rp) * 2 * I * 4);
        p->wb_htq = o; o = align_up(o + nmb * I * rp);
        p->wb_sht = o; o = align_up(o + nmb * mx_groups(rp) * I * 4);
    }
    p->ws_bwd = o;
    return MOE_OK;
}

bool aligned(const void* ptr, size_t a) { return ((uintptr_t)ptr & (a - 1)) == 0; }

// Compute units of the current device (0 if the runtime cannot tell).
int device_cus() {
    int dev = 0, n = 0;
    if (hipGetDevice(&dev) != hipSuccess) return 0;
    if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess) return 0;
    return n;
}

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

// ---------------------------------------------------------------------------
// The allocation-free forward's workspace: this array, one copy per GPU (each
// at its own device address), held from the library's load until the process
// ends.  Host code never passes the array's name to a kernel (on the host it
// is a stand-in, not a device address): it uses the address that
// hipGetSymbolAddress returns on each device, looked up once per device.
// ---------------------------------------------------------------------------
constexpr size_t kStaticWsBytes = (size_t)MOE_STATIC_WORKSPACE_BYTES;
static __device__ __align__(256) uint8_t scratch[kStaticWsBytes];

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices];

// Device address of `scratch` on the current device.
moe_status scratch_address(void** out) {
    int dev = -1;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return MOE_E_HIP;
    std::lock_guard<std::mutex> lock(g_scratch_mu);
    if (!g_scratch_ptr[dev]) {
        void* ptr = nullptr;
        if (hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch)) != hipSuccess || !ptr) return MOE_E_HIP;
        g_scratch_ptr[dev] = ptr;
    }
    *out = g_scratch_ptr[dev];
    return MOE_OK;
}

// The device status word (two ints at the start of a workspace): cleared by a
// kernel (not a memset, so that a captured call records no memset node), and
// copied out to the caller's buffer after the forward.
__global__ void status_clear_kernel(int32_t* word) {
    if (threadIdx.x < 2) word[threadIdx.x] = 0;
}
__global__ void status_copy_kernel(const int32_t* word, int32_t* dst) {
    if (threadIdx.x < 2) dst[threadIdx.x] = word[threadIdx.x];
}

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

moe_status moe_validate_cfg(const moe_cfg* cfg) {
    Plan p;
    return make_plan(cfg, &p);  // the limits that depend on the padded rows too
}

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
    uint16_t* Wdc = (uint16_t*)(base + p.pk_wd);
    uint16_t* Wgu = (uint16_t*)(base + p.pk_wgu);
    launch_pack_gate_up(Wg, Wu, p.E, p.H, p.I, W1t, s);
    launch_transpose(Wd, p.E, p.I, p.H, W2t, s);
    launch_copy(Wd, (size_t)p.E * I * H * 2, Wdc, s);
    launch_concat_gu(Wg, Wu, p.E, p.H, p.I, Wgu, s);
    if (p.mx) {  // E4M3 codes + E8M0 scales along each GEMM's K, expert by expert
        for (int e = 0; e < p.E; ++e) {
            launch_mx_quant(W1t + (size_t)e * 2 * I * H, 2 * p.I, p.H, 1, base + p.pk_w1q + (size_t)e * 2 * I * H,
                            base + p.pk_s1 + (size_t)e * mx_groups(H) * 2 * I * 4, s);
            launch_mx_quant(W2t + (size_t)e * H * I, p.H, p.I, 1, base + p.pk_w2q + (size_t)e * H * I,
                            base + p.pk_s2 + (size_t)e * mx_groups(I) * H * 4, s);
            launch_mx_quant(Wdc + (size_t)e * I * H, p.I, p.H, 1, base + p.pk_wdq + (size_t)e * I * H,
                            base + p.pk_sd + (size_t)e * mx_groups(H) * I * 4, s);
            launch_mx_quant(Wgu + (size_t)e * H * 2 * I, p.H, 2 * p.I, 1, base + p.pk_wguq + (size_t)e * H * 2 * I,
                            base + p.pk_sgu + (size_t)e * mx_groups(2 * I) * H * 4, s);
        }
    }
    if (p.shared) {
        launch_pack_gate_up(Wsg, Wsu, 1, p.H, p.I, W1t + (size_t)p.E * 2 * I * H, s);
        launch_transpose(Wsd, 1, p.I, p.H, W2t + (size_t)p.E * H * I, s);
        launch_copy(Wsd, I * H * 2, Wdc + (size_t)p.E * I * H, s);
        launch_concat_gu(Wsg, Wsu, 1, p.H, p.I, Wgu + (size_t)p.E * H * 2 * I, s);
    }
    return check_launch();
}

moe_status moe_route(const moe_cfg* cfg, const uint16_t* x, const float* Wr, const float* bias,
                     int32_t* topk_idx, float* topk_w, float* logits, uint8_t* x_codes, uint8_t* x_scales,
                     void* stream) {
    moe_status st = validate(cfg);
    if (st != MOE_OK) return st;
    if (!x || !Wr || !topk_idx || !topk_w) return MOE_E_INVALID;
    if ((x_codes == nullptr) != (x_scales == nullptr) || (x_codes && (!aligned(x_codes, 16) || !aligned(x, 16))))
        return MOE_E_INVALID;
    TIMED(MOE_K_ROUTE, (hipStream_t)stream,
          launch_route(x, Wr, bias, cfg->T, cfg->H, cfg->E, cfg->k, topk_idx, topk_w, logits, (hipStream_t)stream,
                       x_codes, x_scales));
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

// Host checks of a forward call's buffers (nothing is enqueued).
static moe_status check_fwd(const Plan& p, const moe_weights* w, const uint16_t* x, const uint16_t* out,
                            const void* saved, size_t saved_bytes, const void* ws, size_t ws_bytes) {
    if (!w || !w->Wr || !w->packed || !x || !out || !ws) return MOE_E_INVALID;
    if (!aligned(x, 16) || !aligned(out, 16) || !aligned(ws, kAlign) || !aligned(w->packed, kAlign))
        return MOE_E_INVALID;
    if (saved && !aligned(saved, kAlign)) return MOE_E_INVALID;
    if (w->packed_bytes < p.packed || ws_bytes < p.ws_fwd) return MOE_E_WORKSPACE;
    if (saved && saved_bytes < p.saved) return MOE_E_WORKSPACE;
    return MOE_OK;
}

// The forward's launches (arguments already checked by check_fwd).
static moe_status enqueue_fwd(const moe_cfg* cfg, const Plan& p, const moe_weights* w, const uint16_t* x,
                              uint16_t* out, void* saved, void* ws, hipStream_t s) {
    uint8_t* wsb = (uint8_t*)ws;
    int32_t* idx = saved ? (int32_t*)((uint8_t*)saved + p.sv_idx) : (int32_t*)(wsb + p.ws_idx);
    float* gw = saved ? (float*)((uint8_t*)saved + p.sv_w) : (float*)(wsb + p.ws_w);
    const uint8_t* pk = (const uint8_t*)w->packed;
    const uint16_t* W1t = (const uint16_t*)(pk + p.pk_w1t);
    const uint16_t* W2t = (const uint16_t*)(pk + p.pk_w2t);
    int32_t* mt_all = (int32_t*)(wsb + p.ws_mt);
    int32_t* prs_all = (int32_t*)(wsb + p.ws_prs);
    int32_t* rows_all = (int32_t*)(wsb + p.ws_rows);
    uint8_t* lay0 = wsb + p.ws_lay0;
    uint8_t* xq = wsb + p.ws_xq;
    uint8_t* sx = wsb + p.ws_sx;
    const int grid = kNumCUs;

    // route every token (under MXFP8 also the dispatch-side quantisation of
    // every token row, along H, from the values the router reads), then lay
    // out every minibatch (one workgroup each)
    const bool quant_x = p.mx && !p.identity;
    TIMED(MOE_K_ROUTE, s, launch_route(x, w->Wr, w->bias, p.T, p.H, p.E, p.k, idx, gw, nullptr, s,
                                       quant_x ? xq : nullptr, quant_x ? sx : nullptr));
    {
        LayoutOut o{};
        o.hdr = (LayoutHeader*)(lay0 + p.ly_hdr);
        o.mt_start = mt_all;
        o.prow_start = prs_all;
        o.prow_token = (int32_t*)(lay0 + p.ly_prow_token);
        o.tok_prow = (int32_t*)(lay0 + p.ly_tok_prow);
        o.rows_e = rows_all;
        o.tok_prow_ld = p.ld_tok_prow;
        LayoutStrides ls{};
        ls.hdr = (int64_t)p.lay_bytes / (int64_t)sizeof(LayoutHeader);
        ls.mt_start = ls.rows_e = ls.prow_start = p.Et + 1;
        ls.prow_token = ls.tok_prow = (int64_t)p.lay_bytes / 4;
        TIMED(MOE_K_LAYOUT, s, launch_layout_batched(idx, p.T, p.Mb, p.E, p.k, p.shared ? 1 : 0, o, ls, s));
    }

    // operands common to every minibatch
    const int e_bf16 = p.mx ? p.E : 0;  // MXFP8 covers the routed experts; bf16 the rest
    GemmArgs g1{};
    g1.A = x; g1.lda = p.H; g1.B = W1t; g1.b_stride = (int64_t)2 * p.I * p.H;
    g1.ldc = p.I; g1.N = 2 * p.I; g1.K = p.H; g1.Et = p.Et; g1.e_begin = e_bf16; g1.e_end = p.Et;
    GemmArgs g2{};
    g2.lda = p.I; g2.B = W2t; g2.b_stride = (int64_t)p.H * p.I;
    g2.ldc = p.H; g2.N = p.H; g2.K = p.I; g2.Et = p.Et; g2.e_begin = e_bf16; g2.e_end = p.Et;
    MxGemmArgs m1{};
    MxGemmArgs m2{};
    if (p.mx) {
        m1.A = xq; m1.lda = p.H; m1.SA = sx; m1.sa_kstride = (int64_t)p.T * 4;
        m1.B = pk + p.pk_w1q; m1.b_stride = (int64_t)2 * p.I * p.H;
        m1.SB = pk + p.pk_s1; m1.sb_stride = mx_groups(p.H) * 2 * p.I * 4; m1.sb_kstride = (int64_t)2 * p.I * 4;
        m1.N = 2 * p.I; m1.K = p.H; m1.e_begin = 0; m1.e_end = p.E; m1.cs_rows = p.rpad;
        m2.lda = p.I; m2.sa_kstride = (int64_t)p.rpad * 4;
        m2.B = pk + p.pk_w2q; m2.b_stride = (int64_t)p.H * p.I;
        m2.SB = pk + p.pk_s2; m2.sb_stride = mx_groups(p.I) * p.H * 4; m2.sb_kstride = (int64_t)p.H * 4;
        m2.N = p.H; m2.K = p.I; m2.e_begin = 0; m2.e_end = p.E; m2.ldc = p.H;
    }

    // one workgroup per CU: the combine workgroups, then a multiple of 8 GEMM
    // workgroups (XCD-aware dealing)
    // Combine tiles with Y in the ring need 3 slots (gate|up(b) waits on
    // combine(b-2) otherwise, which follows it in the tile sequence).
    const int ncu = device_cus();
    const int Sg = p.slots / p.group, ng = ceil_div(p.nmb, p.group);
    const bool ring_ok = ng <= Sg || (Sg >= 2 && (p.comm_cus > 0 || saved || Sg >= 3));
    if (p.mega && ring_ok && ncu >= p.comm_cus + 16) {
        // Training under MXFP8 with the shared expert: the shared expert's two
        // bf16 GEMMs run first, each as one launch over every minibatch,
        // writing its saved g|u, its h and its Y rows; the layer kernel then
        // runs the routed experts' scaled-MFMA tiles only (the instance
        // without bf16 tile code) and its combine adds the shared rows.
        const bool shared_first = p.mx && p.shared && saved != nullptr;
        if (shared_first) {
            uint8_t* sv0 = (uint8_t*)saved + p.sv_mb0;
            GemmArgs ga = g1;  // experts [E, E + 1): the shared expert
            ga.a_row_map = (const int32_t*)(lay0 + p.ly_prow_token); ga.map_mb = (int64_t)p.lay_bytes / 4;
            ga.mt_start = mt_all; ga.prow_start = prs_all; ga.rows_e = rows_all; ga.hdr = nullptr;
            ga.nmb = p.nmb; ga.mt_ld = p.Et + 1;
            ga.C = (uint16_t*)(sv0 + p.sv_hs); ga.c_mb = (int64_t)p.sv_mb / 2;
            ga.GUf = (float*)sv0; ga.gu_mb = (int64_t)p.sv_mb / 4;
            TIMED(MOE_K_SHARED_GEMM, s, launch_grouped_gemm(ga, kEpiSwiGLU, grid, s));
            GemmArgs gb = g2;
            gb.A = (const uint16_t*)(sv0 + p.sv_hs); gb.a_mb = (int64_t)p.sv_mb / 2;
            gb.mt_start = mt_all; gb.prow_start = prs_all; gb.rows_e = rows_all; gb.hdr = nullptr;
            gb.nmb = p.nmb; gb.mt_ld = p.Et + 1;
            gb.C = (uint16_t*)(sv0 + p.sv_y); gb.c_mb = (int64_t)p.sv_mb / 2;
            TIMED(MOE_K_SHARED_GEMM, s, launch_grouped_gemm(gb, kEpiStore, grid, s));
        }
        MegaArgs a{};
        a.T = p.T; a.H = p.H; a.I = p.I; a.k = p.k; a.Mb = p.Mb; a.nmb = p.nmb; a.S = p.slots;
        a.comm = p.comm_cus; a.e_end = shared_first ? p.E : p.Et; a.e_mx = p.mx ? p.E : 0;
        a.with_shared = p.shared ? 1 : 0;
        a.ld_tok_prow = p.ld_tok_prow; a.mx = p.mx ? 1 : 0; a.group = p.group;
        a.lay0 = lay0; a.lay_bytes = p.lay_bytes; a.ly_prow_token = p.ly_prow_token; a.ly_tok_prow = p.ly_tok_prow;
        a.mt_all = mt_all; a.prs_all = prs_all; a.rows_all = rows_all; a.mt_ld = p.Et + 1;
        a.g1 = g1; a.g2 = g2; a.m1 = m1; a.m2 = m2;
        a.g1.e_begin = a.g2.e_begin = 0;
        a.slot0 = wsb + p.ws_slot0; a.slot_bytes = p.slot_bytes;
        a.sl_h = p.sl_h; a.sl_y = p.sl_y; a.sl_hq = p.sl_hq; a.sl_sh = p.sl_sh;
        a.saved_mb0 = saved ? (uint8_t*)saved + p.sv_mb0 : nullptr;
        a.sv_mb = p.sv_mb; a.sv_y = p.sv_y;
        a.gw = gw; a.out = out;
        a.counters = (int*)(wsb + p.ws_cnt);
        a.status = (int*)(wsb + p.ws_status);
        a.spin_ticks = kSpinTicks;
        a.debug_drop = (cfg->flags & MOE_F_DEBUG_DROP_SIGNAL) ? 1 : 0;
        const int mgrid = p.comm_cus + ((ncu - p.comm_cus) / 8) * 8;
        hipError_t err = hipSuccess;
        TIMED(MOE_K_LAYER, s, err = launch_mega(a, mgrid, s));
        if (err != hipSuccess) return MOE_E_HIP;
        return check_launch();
    }

    for (int b = 0; b < p.nmb; ++b) {
        const int t0 = b * p.Mb;
        const int Tm = (p.T - t0) < p.Mb ? (p.T - t0) : p.Mb;
        uint8_t* lay = lay0 + (size_t)b * p.lay_bytes;
        LayoutHeader* hdr = (LayoutHeader*)(lay + p.ly_hdr);
        int32_t* mt = mt_all + (size_t)b * (p.Et + 1);
        int32_t* prs = prs_all + (size_t)b * (p.Et + 1);
        int32_t* prow_token = (int32_t*)(lay + p.ly_prow_token);
        int32_t* tok_prow = (int32_t*)(lay + p.ly_tok_prow);
        uint8_t* slot = wsb + p.ws_slot0 + (size_t)(b % p.slots) * p.slot_bytes;
        uint16_t* hbuf = (uint16_t*)(slot + p.sl_h);
        uint16_t* ybuf = (uint16_t*)(slot + p.sl_y);
        uint16_t* gubuf = nullptr;
        float* guf = nullptr;
        if (saved) {  // keep g|u and Y of every minibatch for the backward
            uint8_t* mb = (uint8_t*)saved + p.sv_mb0 + (size_t)b * p.sv_mb;
            if (p.mx)
                guf = (float*)mb;
            else
                gubuf = (uint16_t*)mb;
            ybuf = (uint16_t*)(mb + p.sv_y);
        }

        if (p.identity) {
            TIMED(MOE_K_GATHER, s, launch_gather_rows(x, p.H, prow_token, hdr, (int)p.rpad, ybuf, p.H, s));
        } else {
            if (p.mx) {
                MxGemmArgs m = m1;
                m.a_row_map = prow_token; m.mt_start = mt; m.prow_start = prs; m.hdr = hdr;
                m.Cq = slot + p.sl_hq; m.Cs = slot + p.sl_sh; m.GU = guf; m.rows_e = rows_all + (size_t)b * (p.Et + 1);
                TIMED(MOE_K_GEMM_GATE_UP, s, launch_mx_gemm(m, kEpiSwiGLU, grid, s));
            }
            GemmArgs ga = g1;
            ga.a_row_map = prow_token; ga.mt_start = mt; ga.prow_start = prs; ga.hdr = hdr; ga.rows_e = rows_all + (size_t)b * (p.Et + 1);
            ga.C = hbuf; ga.GU = gubuf; ga.GUf = guf;
            if (e_bf16 < p.Et)
                TIMED(p.mx ? MOE_K_SHARED_GEMM : MOE_K_GEMM_GATE_UP, s, launch_grouped_gemm(ga, kEpiSwiGLU, grid, s));
            if (p.mx) {
                MxGemmArgs m = m2;
                m.A = slot + p.sl_hq; m.SA = slot + p.sl_sh; m.mt_start = mt; m.prow_start = prs; m.hdr = hdr;
                m.C = ybuf;
                m.rows_e = rows_all + (size_t)b * (p.Et + 1);
                TIMED(MOE_K_GEMM_DOWN, s, launch_mx_gemm(m, kEpiStore, grid, s));
            }
            GemmArgs gb = g2;
            gb.A = hbuf; gb.mt_start = mt; gb.prow_start = prs; gb.hdr = hdr; gb.C = ybuf; gb.rows_e = rows_all + (size_t)b * (p.Et + 1);
            if (e_bf16 < p.Et)
                TIMED(p.mx ? MOE_K_SHARED_GEMM : MOE_K_GEMM_DOWN, s, launch_grouped_gemm(gb, kEpiStore, grid, s));
        }
        TIMED(MOE_K_COMBINE, s,
              launch_combine(ybuf, p.H, tok_prow, p.ld_tok_prow, gw + (size_t)t0 * p.k, p.k,
                             (p.shared && !p.identity) ? 1 : 0, p.H, Tm, out + (size_t)t0 * p.H, s));
    }
    return check_launch();
}

moe_status moe_layer_fwd(const moe_cfg* cfg, const moe_weights* w, const uint16_t* x, uint16_t* out,
                         void* saved, size_t saved_bytes, void* ws, size_t ws_bytes, void* stream) {
    Plan p;
    moe_status st = make_plan(cfg, &p);
    if (st != MOE_OK) return st;
    if ((st = check_fwd(p, w, x, out, saved, saved_bytes, ws, ws_bytes)) != MOE_OK) return st;
    return enqueue_fwd(cfg, p, w, x, out, saved, ws, (hipStream_t)stream);
}

moe_status moe_layer_fwd_static(const moe_cfg* cfg, const moe_weights* w, const uint16_t* x, uint16_t* out,
                                int32_t* status, void* stream) {
    Plan p;
    moe_status st = make_plan(cfg, &p);
    if (st != MOE_OK) return st;
    if (p.ws_fwd > kStaticWsBytes) return MOE_E_WORKSPACE;  // before any device call
    if (status && !aligned(status, 4)) return MOE_E_INVALID;
    void* ws = nullptr;
    if ((st = scratch_address(&ws)) != MOE_OK) return st;
    if ((st = check_fwd(p, w, x, out, nullptr, 0, ws, kStaticWsBytes)) != MOE_OK) return st;
    hipStream_t s = (hipStream_t)stream;
    hipLaunchKernelGGL(status_clear_kernel, dim3(1), dim3(64), 0, s, (int32_t*)ws);
    if ((st = enqueue_fwd(cfg, p, w, x, out, nullptr, ws, s)) != MOE_OK) return st;
    if (status) hipLaunchKernelGGL(status_copy_kernel, dim3(1), dim3(64), 0, s, (const int32_t*)ws, status);
    return check_launch();
}

moe_status moe_layer_bwd(const moe_cfg* cfg, const moe_weights* w, const uint16_t* x, const uint16_t* dout,
                         const void* saved, size_t saved_bytes, uint16_t* dx, float* dWg, float* dWu,
                         float* dWd, float* dWr, float* dWs, float* dgate, void* ws, size_t ws_bytes,
                         void* stream) {
    Plan p;
    moe_status st = make_plan(cfg, &p);
    if (st != MOE_OK) return st;
    if (p.identity) return MOE_E_UNSUPPORTED;
    if (!w || !w->Wr || !w->packed || !x || !dout || !saved || !dx || !dWg || !dWu || !dWd || !dWr || !ws)
        return MOE_E_INVALID;
    if (p.shared && !dWs) return MOE_E_INVALID;
    if (!aligned(x, 16) || !aligned(dout, 16) || !aligned(dx, 16) || !aligned(ws, kAlign) ||
        !aligned(saved, kAlign) || !aligned(w->packed, kAlign) || !aligned(w->Wr, 16))
        return MOE_E_INVALID;
    if (w->packed_bytes < p.packed || saved_bytes < p.saved || ws_bytes < p.ws_bwd) return MOE_E_WORKSPACE;
    hipStream_t s = (hipStream_t)stream;
    const int E = p.E, H = p.H, I = p.I, k = p.k, Et = p.Et;
    const int64_t rp = p.rpad;
    const uint8_t* sv = (const uint8_t*)saved;
    const int32_t* idx = (const int32_t*)(sv + p.sv_idx);
    const float* gw = (const float*)(sv + p.sv_w);
    const uint8_t* pk = (const uint8_t*)w->packed;
    const uint16_t* Wdc = (const uint16_t*)(pk + p.pk_wd);
    const uint16_t* Wgu = (const uint16_t*)(pk + p.pk_wgu);
    uint8_t* wsb = (uint8_t*)ws;
    float* WrT = (float*)(wsb + p.wb_wrt);
    int32_t* mt_all = (int32_t*)(wsb + p.wb_mt);
    int32_t* prs_all = (int32_t*)(wsb + p.wb_prs);
    uint16_t* dGU_all = (uint16_t*)(wsb + p.wb_dgu);
    uint16_t* HW_all = (uint16_t*)(wsb + p.wb_hw);
    float* dsel_all = (float*)(wsb + p.wb_dsel);
    uint16_t* dH = (uint16_t*)(wsb + p.wb_dh);
    uint16_t* dXb = (uint16_t*)(wsb + p.wb_dx);
    float* dgp = (float*)(wsb + p.wb_dgp);
    float* roww = (float*)(wsb + p.wb_roww);
    const int grid = kNumCUs;

    TIMED(MOE_K_OTHER, s, launch_transpose_f32(w->Wr, H, E, WrT, s));
    {  // every minibatch's layout, with the slot of each padded row
        uint8_t* lay0 = wsb + p.wb_lay0;
        LayoutOut o{};
        o.hdr = (LayoutHeader*)(lay0 + p.ly_hdr);
        o.mt_start = mt_all;
        o.prow_start = prs_all;
        o.prow_token = (int32_t*)(lay0 + p.ly_prow_token);
        o.tok_prow = (int32_t*)(lay0 + p.ly_tok_prow);
        o.prow_slot = (int32_t*)(lay0 + p.ly_prow_slot);
        o.rows_e = (int32_t*)(wsb + p.wb_rows);
        o.tok_prow_ld = p.ld_tok_prow;
        LayoutStrides ls{};
        ls.hdr = (int64_t)p.lay_bytes / (int64_t)sizeof(LayoutHeader);
        ls.mt_start = ls.rows_e = ls.prow_start = Et + 1;
        ls.prow_token = ls.tok_prow = ls.prow_slot = (int64_t)p.lay_bytes / 4;
        TIMED(MOE_K_LAYOUT, s, launch_layout_batched(idx, p.T, p.Mb, E, k, p.shared ? 1 : 0, o, ls, s));
    }
    // The backward runs in phases over chunks of minibatches: reverse-combine
    // of each minibatch of the chunk, one launch of the down input-gradient
    // GEMM over all of them, the SwiGLU backward of each, one launch of the
    // gate|up input-gradient GEMM, then the reverse-dispatch of each (a GEMM
    // launch then has one partial last wave of tiles per chunk instead of one
    // per minibatch).  The per-minibatch buffers hold one chunk; minibatch b
    // uses copy b - b0.
    const int e_bf16 = p.mx ? E : 0;  // MXFP8: experts [0, E) on the scaled-MFMA kernel, the shared expert bf16
    // weight gradients: under MXFP8 ones experts [0, E) on the scaled-MFMA
    // kernel, the shared expert (if any) on the bf16 one
    const int w_bf16 = p.mxw ? E : 0;
    const int32_t* rows_all = (const int32_t*)(wsb + p.wb_rows);
    const int64_t nhb = H / 64;
    float* dHf = p.mx ? (float*)dH : nullptr;  // fp32 under MXFP8
    auto lay_of = [&](int b) { return wsb + p.wb_lay0 + (size_t)b * p.lay_bytes; };
    for (int b0 = 0; b0 < p.nmb; b0 += p.bchunk) {
        const int b1 = (b0 + p.bchunk) < p.nmb ? b0 + p.bchunk : p.nmb;
        const int32_t* mt_c = mt_all + (size_t)b0 * (Et + 1);
        const int32_t* prs_c = prs_all + (size_t)b0 * (Et + 1);
        const int32_t* rows_c = rows_all + (size_t)b0 * (Et + 1);
        for (int b = b0; b < b1; ++b) {
            const size_t j = (size_t)(b - b0);
            uint8_t* lay = lay_of(b);
            const uint8_t* svb = sv + p.sv_mb0 + (size_t)b * p.sv_mb;
            RcombArgs rc{};
            rc.dout = dout; rc.x = x; rc.Y = (const uint16_t*)(svb + p.sv_y); rc.topk_w = gw;
            rc.prow_token = (int32_t*)(lay + p.ly_prow_token);
            rc.prow_slot = (int32_t*)(lay + p.ly_prow_slot); rc.hdr = (LayoutHeader*)(lay + p.ly_hdr);
            rc.row_w = roww + j * rp;
            rc.dgp = dgp + j * rp * nhb; rc.dsel = dsel_all + (size_t)b * rp;
            rc.H = H; rc.k = k; rc.nhb = (int)nhb; rc.ldt = rp;
            // MXFP8: dY quantised from fp32 here (along H, the down input-gradient GEMM's K)
            rc.dYq = p.mx ? wsb + p.wb_dyq + j * rp * H : nullptr;
            rc.sdY = p.mx ? wsb + p.wb_sdy + j * mx_groups(H) * rp * 4 : nullptr;
            rc.dyq_row_end = prs_all + (size_t)b * (Et + 1) + e_bf16;
            if (p.mxw) {  // weight-gradient operands of the MXFP8 experts (rows before dyq_row_end)
                rc.dYTq = wsb + p.wb_dytq + (size_t)b * H * rp;
                rc.sdYT = wsb + p.wb_sdyt + (size_t)b * mx_groups(rp) * H * 4;
                rc.xgTq = wsb + p.wb_xgtq + (size_t)b * H * rp;
                rc.sxgT = wsb + p.wb_sxgt + (size_t)b * mx_groups(rp) * H * 4;
            }
            TIMED(MOE_K_GATHER, s, launch_rcomb_gather(rc, (int)rp, s));
        }
        if (p.mx) {
            MxGemmArgs m1{};  // dH = Q(dY) Q(Wd)^T
            m1.A = wsb + p.wb_dyq; m1.a_row_map = nullptr; m1.lda = H;
            m1.SA = wsb + p.wb_sdy; m1.sa_kstride = rp * 4;
            m1.B = pk + p.pk_wdq; m1.b_stride = (int64_t)I * H;
            m1.SB = pk + p.pk_sd; m1.sb_stride = mx_groups(H) * I * 4; m1.sb_kstride = (int64_t)I * 4;
            m1.N = I; m1.K = H; m1.mt_start = mt_c; m1.prow_start = prs_c; m1.hdr = nullptr; m1.e_begin = 0; m1.e_end = E;
            m1.C = nullptr; m1.ldc = I; m1.Cq = nullptr; m1.Cs = nullptr; m1.cs_rows = 0; m1.GU = nullptr;
            m1.Cf = dHf; m1.rows_e = rows_c;
            m1.nmb = b1 - b0; m1.mt_ld = Et + 1; m1.a_mb = rp * H; m1.sa_mb = mx_groups(H) * rp * 4; m1.c_mb = rp * I;
            TIMED(MOE_K_DGRAD_DOWN, s, launch_mx_gemm(m1, kEpiStore, grid, s));
        }
        if (e_bf16 < Et) {
            // dH = dY Wd^T with dY_r = w_r dout[t_r]: the gathered dout rows
            // times Wd^T, each output row scaled by w_r (1 for the shared expert)
            GemmArgs g1{};
            g1.A = dout; g1.a_row_map = (const int32_t*)(lay_of(b0) + p.ly_prow_token);
            g1.map_mb = (int64_t)p.lay_bytes / 4;
            g1.row_scale = roww; g1.rs_mb = rp;
            g1.lda = H;
            g1.B = Wdc; g1.b_stride = (int64_t)I * H;
            g1.C = dH; g1.ldc = I; g1.N = I; g1.K = H;
            g1.mt_start = mt_c; g1.prow_start = prs_c; g1.hdr = nullptr; g1.Et = Et; g1.GU = nullptr; g1.e_begin = e_bf16; g1.e_end = Et;
            g1.GUf = nullptr; g1.Cf = dHf; g1.rows_e = rows_c;
            g1.nmb = b1 - b0; g1.mt_ld = Et + 1; g1.c_mb = rp * I;
            TIMED(p.mx ? MOE_K_SHARED_GEMM : MOE_K_DGRAD_DOWN, s, launch_grouped_gemm(g1, kEpiStore, grid, s));
        }
        for (int b = b0; b < b1; ++b) {
            const size_t j = (size_t)(b - b0);
            uint8_t* lay = lay_of(b);
            const uint8_t* svb = sv + p.sv_mb0 + (size_t)b * p.sv_mb;
            const size_t bh = j * rp * I;  // this minibatch's dH elements
            SwigluBwdArgs sb{};
            sb.dH = p.mx ? nullptr : dH + bh; sb.GU = (const uint16_t*)svb; sb.hdr = (LayoutHeader*)(lay + p.ly_hdr);
            sb.row_w = roww + j * rp;
            sb.dGU = dGU_all + (size_t)b * rp * 2 * I; sb.HW = HW_all + (size_t)b * rp * I;
            sb.dgu_row0 = prs_all + (size_t)b * (Et + 1) + w_bf16;  // bf16 weight gradients: row 0 (every row)
            sb.I = I; sb.ldt = rp;
            // MXFP8: fp32 inputs, dG|dU quantised here (along I, the gate|up input-gradient GEMM's K)
            sb.dHf = p.mx ? dHf + bh : nullptr; sb.GUf = p.mx ? (const float*)svb : nullptr;
            sb.dGUq = p.mx ? wsb + p.wb_dguq + 2 * bh : nullptr;
            sb.sdGU = p.mx ? wsb + p.wb_sdgu + j * mx_groups(2 * I) * rp * 4 : nullptr;
            if (p.mxw) {  // weight-gradient operands of the MXFP8 experts (rows before dgu_row0)
                sb.prow_slot = (const int32_t*)(lay + p.ly_prow_slot);
                sb.dGUTq = wsb + p.wb_dgutq + (size_t)b * 2 * I * rp;
                sb.sdGUT = wsb + p.wb_sdgut + (size_t)b * mx_groups(rp) * 2 * I * 4;
                sb.HTq = wsb + p.wb_htq + (size_t)b * I * rp;
                sb.sHT = wsb + p.wb_sht + (size_t)b * mx_groups(rp) * I * 4;
            }
            TIMED(MOE_K_GATHER, s, launch_swiglu_bwd(sb, (int)rp, s));
        }
        if (p.mx) {
            MxGemmArgs m2{};  // dX = Q(dG | dU) Q(Wg | Wu)^T
            m2.A = wsb + p.wb_dguq; m2.a_row_map = nullptr; m2.lda = 2 * I;
            m2.SA = wsb + p.wb_sdgu; m2.sa_kstride = rp * 4;
            m2.B = pk + p.pk_wguq; m2.b_stride = (int64_t)H * 2 * I;
            m2.SB = pk + p.pk_sgu; m2.sb_stride = mx_groups(2 * I) * H * 4; m2.sb_kstride = (int64_t)H * 4;
            m2.N = H; m2.K = 2 * I; m2.mt_start = mt_c; m2.prow_start = prs_c; m2.hdr = nullptr; m2.e_begin = 0; m2.e_end = E;
            m2.C = dXb; m2.ldc = H; m2.Cq = nullptr; m2.Cs = nullptr; m2.cs_rows = 0; m2.GU = nullptr;
            m2.Cf = nullptr; m2.rows_e = rows_c;
            m2.nmb = b1 - b0; m2.mt_ld = Et + 1; m2.a_mb = rp * 2 * I; m2.sa_mb = mx_groups(2 * I) * rp * 4; m2.c_mb = rp * H;
            TIMED(MOE_K_DGRAD_GATE_UP, s, launch_mx_gemm(m2, kEpiStore, grid, s));
        }
        if (e_bf16 < Et) {
            GemmArgs g2{};  // dX = dG Wg^T + dU Wu^T
            g2.A = dGU_all + (size_t)b0 * rp * 2 * I; g2.a_row_map = nullptr; g2.lda = 2 * I;
            g2.B = Wgu; g2.b_stride = (int64_t)H * 2 * I;
            g2.C = dXb; g2.ldc = H; g2.N = H; g2.K = 2 * I;
            g2.mt_start = mt_c; g2.prow_start = prs_c; g2.hdr = nullptr; g2.Et = Et;
            g2.GU = nullptr; g2.e_begin = e_bf16; g2.e_end = Et; g2.GUf = nullptr; g2.Cf = nullptr;
            g2.rows_e = rows_c;
            g2.nmb = b1 - b0; g2.mt_ld = Et + 1; g2.a_mb = rp * 2 * I; g2.c_mb = rp * H;
            TIMED(p.mx ? MOE_K_SHARED_GEMM : MOE_K_DGRAD_GATE_UP, s, launch_grouped_gemm(g2, kEpiStore, grid, s));
        }
        for (int b = b0; b < b1; ++b) {
            const size_t j = (size_t)(b - b0);
            const int t0 = b * p.Mb;
            const int Tm = (p.T - t0) < p.Mb ? (p.T - t0) : p.Mb;
            uint8_t* lay = lay_of(b);
            RdispArgs rd{};
            rd.dX = dXb + j * rp * H; rd.dgp = dgp + j * rp * nhb;
            rd.tok_prow = (int32_t*)(lay + p.ly_tok_prow); rd.topk_idx = idx; rd.topk_w = gw; rd.WrT = WrT;
            rd.dsel = dsel_all + (size_t)b * rp; rd.dgate = dgate; rd.dx = dx; rd.t0 = t0; rd.H = H; rd.k = k;
            rd.ld = p.ld_tok_prow; rd.with_shared = p.shared ? 1 : 0; rd.nhb = (int)nhb;
            rd.dlogits = (float*)(wsb + p.wb_dlog); rd.E = E;
            TIMED(MOE_K_COMBINE, s, launch_rdispatch(rd, Tm, s));
        }
    }
    if (p.mxw) {
        MxWgradArgs qa{};  // [dWg | dWu][e] = Q(x_e)^T Q([dG | dU]_e)
        qa.A = wsb + p.wb_xgtq; qa.SA = wsb + p.wb_sxgt; qa.B = wsb + p.wb_dgutq; qa.SB = wsb + p.wb_sdgut;
        qa.ld = rp; qa.a_mb = (int64_t)H * rp; qa.b_mb = (int64_t)2 * I * rp;
        qa.sa_mb = mx_groups(rp) * H * 4; qa.sb_mb = mx_groups(rp) * 2 * I * 4;
        qa.M = H; qa.N = 2 * I; qa.n_split = I; qa.E = E; qa.nmb = p.nmb; qa.mt_ld = Et + 1;
        qa.prs = prs_all; qa.rows = rows_all; qa.C0 = dWg; qa.C1 = dWu;
        TIMED(MOE_K_WGRAD, s, launch_mx_wgrad(qa, grid, s));
        MxWgradArgs qd{};  // dWd[e] = Q(h_e)^T Q(dY_e)
        qd.A = wsb + p.wb_htq; qd.SA = wsb + p.wb_sht; qd.B = wsb + p.wb_dytq; qd.SB = wsb + p.wb_sdyt;
        qd.ld = rp; qd.a_mb = (int64_t)I * rp; qd.b_mb = (int64_t)H * rp;
        qd.sa_mb = mx_groups(rp) * I * 4; qd.sb_mb = mx_groups(rp) * H * 4;
        qd.M = I; qd.N = H; qd.n_split = H; qd.E = E; qd.nmb = p.nmb; qd.mt_ld = Et + 1;
        qd.prs = prs_all; qd.rows = rows_all; qd.C0 = dWd; qd.C1 = nullptr;
        TIMED(MOE_K_WGRAD, s, launch_mx_wgrad(qd, grid, s));
    }
    if (w_bf16 < Et) {
        // row -> token maps of the minibatches: the gathered operands x and dout
        const int32_t* map0 = (const int32_t*)(lay_of(0) + p.ly_prow_token);
        const int64_t map_mb = (int64_t)p.lay_bytes / 4;
        WgradArgs wa{};  // [dWg | dWu][e] = x_e^T [dG | dU]_e over every row of expert e
        wa.A = x; wa.lda = H; wa.gather = 1; wa.map = map0; wa.map_mb = map_mb;
        wa.B = dGU_all; wa.ldb = 2 * I; wa.b_mb = rp * 2 * I;
        wa.M = H; wa.N = 2 * I; wa.n_split = I; wa.Et = Et; wa.e_begin = w_bf16; wa.nmb = p.nmb; wa.mt_ld = Et + 1;
        wa.prs = prs_all; wa.rows = rows_all;
        wa.C0 = dWg; wa.C1 = dWu;
        wa.Cs0 = p.shared ? dWs : nullptr; wa.Cs1 = p.shared ? dWs + (size_t)H * I : nullptr;
        TIMED(p.mxw ? MOE_K_SHARED_GEMM : MOE_K_WGRAD, s, launch_wgrad(wa, grid, s));
        WgradArgs wd{};  // dWd[e] = h_e^T dY_e = (w h)_e^T dout[t_r]
        wd.A = HW_all; wd.lda = I; wd.a_mb = rp * I;
        wd.B = dout; wd.ldb = H; wd.gather = 2; wd.map = map0; wd.map_mb = map_mb;
        wd.M = I; wd.N = H; wd.n_split = H; wd.Et = Et; wd.e_begin = w_bf16; wd.nmb = p.nmb; wd.mt_ld = Et + 1;
        wd.prs = prs_all; wd.rows = rows_all;
        wd.C0 = dWd; wd.C1 = nullptr;
        wd.Cs0 = p.shared ? dWs + (size_t)2 * H * I : nullptr; wd.Cs1 = nullptr;
        TIMED(p.mxw ? MOE_K_SHARED_GEMM : MOE_K_WGRAD, s, launch_wgrad(wd, grid, s));
    }
    DwrArgs dr{};
    dr.x = x; dr.dlogits = (const float*)(wsb + p.wb_dlog); dr.partial = (float*)(wsb + p.wb_dwrp);
    dr.dWr = dWr; dr.T = p.T; dr.H = H; dr.E = E;
    TIMED(MOE_K_OTHER, s, launch_dwr(dr, s));
    return check_launch();
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

moe_status moe_mx_quantize(const uint16_t* src, int64_t rows, int32_t cols, uint8_t* codes, uint8_t* scales,
                           void* stream) {
    if (!src || !codes || !scales || rows < 1 || cols < 32) return MOE_E_INVALID;
    if (cols % 32 || !aligned(src, 16) || !aligned(codes, 16)) return MOE_E_INVALID;
    launch_mx_quant(src, rows, cols, 0, codes, scales, (hipStream_t)stream);
    return check_launch();
}

// Destroys every timing event (they must not outlive the runtime's own
// teardown at process exit, which runs after profiling tools have finalised).
static moe_status release_timing_events() {
    moe_status st = MOE_OK;
    for (hipEvent_t e : g_timing.ev)
        if (e && hipEventDestroy(e) != hipSuccess) st = MOE_E_HIP;
    g_timing.ev.clear();
    g_timing.kind.clear();
    g_timing.used = 0;
    return st;
}

moe_status moe_timing_enable(int32_t on) {
    if (!on) {
        // the recorded pairs may still be pending on their streams: wait for
        // them before the events go
        for (int i = 0; i < g_timing.used; ++i) (void)hipEventSynchronize(g_timing.ev[2 * i + 1]);
        g_timing.on = false;
        return release_timing_events();
    }
    if (g_timing.ev.empty()) {
        g_timing.ev.assign(2 * kTimingPairs, nullptr);
        g_timing.kind.resize(kTimingPairs);
        for (auto& e : g_timing.ev)
            if (hipEventCreate(&e) != hipSuccess) {
                release_timing_events();
                return MOE_E_HIP;
            }
    }
    g_timing.used = 0;
    g_timing.dropped = 0;
    g_timing.on = true;
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
