// C ABI of the parallel-drafting step: argument checks, the handle's scratch,
// the launch sequence of one drafter pass, status word and event timing.
//
// [Blog] = "P-EAGLE: Faster LLM Inference with Parallel Speculative Decoding
// in vLLM" (summary page); [Paper] = "P-EAGLE: Parallel-Drafting EAGLE with
// Scalable Training" (summary page); [arXiv] = its ScienceStack page.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <cmath>
#include <cstdlib>
#include <cstring>
#include <mutex>
#include <new>
#include <utility>
#include <vector>

#include "kernels.hpp"
#include "pd.h"

using namespace pd;

struct pd_handle {
    int device = -1;
    char* scratch = nullptr;
    size_t scratch_bytes = 0;
    int32_t* status = nullptr;
    float* dbg = nullptr;
    uint64_t* timeline = nullptr;   // decode kernel phase timestamps, or null
    int prof = 0;  // bit mask of recorded kernel classes
    std::vector<std::pair<hipEvent_t, hipEvent_t>> ev[PD_KERNEL_CLASSES];
    std::vector<hipEvent_t> spare;
};

// Scratch of the allocation-free forward (pd_draft_forward_noalloc): one
// array per device, held until the process ends. In host code `scratch` only
// names the symbol; its device address comes from hipGetSymbolAddress, taken
// once per device with that device current, and only that address is ever
// passed to kernels or copies.
constexpr size_t kStaticScratchBytes = PD_NOALLOC_SCRATCH_BYTES;
static __device__ __align__(256) char scratch[kStaticScratchBytes];

namespace {

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
char* g_scratch_ptr[kMaxDevices] = {};

// The current device's scratch address (looked up on its first use).
int static_scratch(char** out) {
    int dev = -1;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return PD_EHIP;
    std::lock_guard<std::mutex> lock(g_scratch_mu);
    if (!g_scratch_ptr[dev]) {
        void* ptr = nullptr;
        if (hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch)) != hipSuccess || !ptr) return PD_EHIP;
        g_scratch_ptr[dev] = static_cast<char*>(ptr);
    }
    *out = g_scratch_ptr[dev];
    return PD_OK;
}

constexpr int kMaxTin = 1 << 20;

size_t align256(size_t x) { return (x + 255) & ~size_t(255); }

bool dims_ok(const pd_batch_dims* d) {
    if (!d) return false;
    if (d->C < 0 || d->C > PD_MAX_C) return false;
    if (d->K < 1 || d->K > PD_MAX_K) return false;
    if (d->T_in < d->C || d->T_in > kMaxTin) return false;
    if (d->hidden3 <= 0 || d->hidden3 % 8 != 0) return false;
    if (d->block_size < 1 || d->max_blocks < 1 || d->num_blocks < 1) return false;
    if ((long long)d->num_blocks * d->block_size > (1LL << 31) - 1) return false;
    if ((long long)d->max_blocks * d->block_size > (1LL << 30)) return false;
    return true;
}

hipEvent_t take_event(pd_handle* h) {
    if (!h->spare.empty()) {
        hipEvent_t e = h->spare.back();
        h->spare.pop_back();
        return e;
    }
    hipEvent_t e = nullptr;
    if (hipEventCreate(&e) != hipSuccess) return nullptr;
    return e;
}

// Event pair around one launch when profiling is on.
struct Timed {
    pd_handle* h;
    int cls;
    hipStream_t s;
    hipEvent_t e0 = nullptr, e1 = nullptr;
    Timed(pd_handle* h_, int cls_, hipStream_t s_) : h(h_), cls(cls_), s(s_) {
        if (h && (h->prof & (1 << cls))) {
            e0 = take_event(h);
            e1 = take_event(h);
            if (e0 && e1) (void)hipEventRecord(e0, s);
        }
    }
    ~Timed() {
        if (e0 && e1) {
            (void)hipEventRecord(e1, s);
            h->ev[cls].emplace_back(e0, e1);
        }
    }
};

struct Layout {
    size_t sync, x, u, q, ao, act, ws, po, pml, plan, xg, amv, ami, total;
    // row compaction (compact): gathered hidden rows, ids, positions, slots,
    // row map, request starts, sampled-row indices, {kept rows, split count}
    size_t hid_c, ids_c, pos_c, slot_c, rowmap, cu_c, nti_c, cnt;
    bool compact;
    int T, R, ntilesV;   // ntilesV: argmax partials per row of the LM-head GEMM kernel
    int amax_cap;        // partials per row the scratch holds (also the decode pass's)
    AttnSplit sp;
    DecodePlan dp;   // the persistent decode pass, when it applies (dp.ok)
};

// Passes of more than 64 rows compute only their rows that are not rejected
// (gathered to the front by a compaction launch, counted on the device);
// PD_COMPACT=0 in the environment computes every row instead.
bool compact_enabled() {
    const char* e = std::getenv("PD_COMPACT");
    return !(e && e[0] == '0');
}

// The persistent decode kernel serves passes of up to 64 rows when the
// environment sets PD_DECODE=1; otherwise every pass runs as separate
// kernels (measured faster so far).
bool decode_enabled() {
    const char* e = std::getenv("PD_DECODE");
    return e && e[0] == '1';
}

// limit != 0: the attention partial planes (sized by the splits per request,
// scap) shrink until the whole layout fits in `limit` bytes; fewer splits per
// request only make the device plan pick longer splits. L.total > limit when
// even the fewest splits the block table needs do not fit.
// hidden_d: the caller gives the projected hidden rows (no fc projection).
Layout plan_layout(const pd_model* m, const pd_batch_dims* d, bool fp8, bool hidden_d, size_t limit = 0) {
    Layout L;
    const int T = d->T_in + d->C * (d->K - 1);
    const int R = d->C * d->K;
    L.T = T;
    L.R = R;
    const int qkvw = (m->Hq + 2 * m->Hkv) * m->dh;
    const int hd = m->Hq * m->dh;
    L.sp = plan_attn_split(d->C, T, m->Hq, m->Hkv, m->dh, d->max_blocks);
    L.compact = compact_enabled() && T > 64 && T <= kCompactMaxRows && !hidden_d;
    size_t ws = 0;
    auto need = [&](int M, int N, int K) {
        GemmPlan p = plan_gemm(M, N, K, EPI_PARTIAL, L.compact);
        ws = std::max(ws, gemm_ws_floats(p, M, N, EPI_PARTIAL));
    };
    auto need_all = [&]() {
        ws = 0;
        need(T, m->d, m->hidden3);
        need(T, qkvw, 2 * m->d);
        need(T, qkvw, m->d);
        need(T, m->d, hd);
        need(T, m->d, m->F);
    };
    need_all();
    L.ntilesV = plan_lm_head(R, m->V, m->d).ntiles;
    L.amax_cap = L.ntilesV;
    L.dp = plan_decode(*m, T, R, fp8);
    if (!decode_enabled()) L.dp.ok = false;
    int u_slots = 1, l_slots = 1;   // activation slots (the decode pass writes each once)
    if (L.dp.ok) {
        ws = std::max(ws, L.dp.ws_floats);
        L.amax_cap = std::max(L.amax_cap, L.dp.lm_ntiles);
        L.sp = plan_attn_split_grid(d->C, T, m->Hq, m->Hkv, m->dh, d->max_blocks, L.dp.grid);
        u_slots = 2 * m->N;
        l_slots = m->N;
    }
    auto carve_all = [&]() {
        size_t off = 0;
        auto carve = [&](size_t bytes) { size_t o = off; off += align256(bytes); return o; };
        // barrier words of the decode kernel: always first, so that no other
        // use of the scratch ever writes them (they must start at zero)
        L.sync = carve(kDecodeSyncWords * 4);
        L.x = carve((size_t)T * m->d * 4);
        L.u = carve((size_t)u_slots * T * 2 * m->d * 2);
        L.q = carve((size_t)T * hd * 2);
        L.ao = carve((size_t)l_slots * T * hd * 2);
        L.act = carve((size_t)l_slots * T * m->F * 2);
        L.ws = carve(ws * 4);
        L.po = carve((size_t)L.sp.scap * T * hd * 4);
        L.pml = carve((size_t)L.sp.scap * T * m->Hq * 2 * 4);
        L.plan = carve(attn_plan_ints(L.sp) * 4);
        L.xg = carve((size_t)R * m->d * 2);
        L.amv = carve((size_t)R * L.amax_cap * 4);
        L.ami = carve((size_t)R * L.amax_cap * 4);
        const int tc = L.compact ? T : 0;
        L.hid_c = carve((size_t)tc * m->hidden3 * 2);
        L.ids_c = carve((size_t)tc * 4);
        L.pos_c = carve((size_t)tc * 4);
        L.slot_c = carve((size_t)tc * 4);
        L.rowmap = carve((size_t)tc * 4);
        L.cu_c = carve(L.compact ? (size_t)(d->C + 1) * 4 : 0);
        L.nti_c = carve(L.compact ? (size_t)R * 4 : 0);
        L.cnt = carve(L.compact ? 2 * 4 : 0);
        L.total = off;
    };
    carve_all();
    if (limit && L.total > limit && L.compact) {   // the bounded scratch: every row computed
        L.compact = false;
        need_all();
        if (L.dp.ok) ws = std::max(ws, L.dp.ws_floats);
        carve_all();
    }
    if (limit && L.total > limit) {
        const size_t per_split = align256((size_t)T * hd * 4) + align256((size_t)T * m->Hq * 2 * 4);
        const size_t fixed = L.total - (size_t)L.sp.scap * per_split;   // upper bound: alignment slack
        const int need = attn_min_splits(d->max_blocks);
        const long long fit = fixed < limit ? (long long)((limit - fixed) / per_split) : 0;
        if (fit >= need && fit < L.sp.scap) {
            L.sp.scap = (int)fit;
            carve_all();
        }
    }
    return L;
}

int ensure_scratch(pd_handle* h, size_t bytes, hipStream_t s) {
    if (h->scratch_bytes >= bytes) return PD_OK;
    if (h->scratch) {
        (void)hipStreamSynchronize(s);
        (void)hipFree(h->scratch);
        h->scratch = nullptr;
        h->scratch_bytes = 0;
    }
    const size_t want = bytes + bytes / 4;
    if (hipMalloc(&h->scratch, want) != hipSuccess) {
        h->scratch = nullptr;
        return PD_ENOMEM;
    }
    h->scratch_bytes = want;
    // the decode kernel's barrier words start at zero (scratch offset 0)
    if (hipMemsetAsync(h->scratch, 0, kDecodeSyncWords * 4, s) != hipSuccess) return PD_EHIP;
    return PD_OK;
}

int create_handle(pd_handle** out) {
    pd_handle* h = new (std::nothrow) pd_handle();
    if (!h) return PD_ENOMEM;
    (void)hipGetDevice(&h->device);
    if (hipMalloc(&h->status, sizeof(int32_t)) != hipSuccess) {
        pd_free(h);
        return PD_ENOMEM;
    }
    if (hipMemset(h->status, 0, sizeof(int32_t)) != hipSuccess ||
        hipDeviceSynchronize() != hipSuccess) {
        pd_free(h);
        return PD_EHIP;
    }
    *out = h;
    return PD_OK;
}

bool model_ok(const pd_model* m) {
    if (!m) return false;
    if (m->d <= 0 || m->d % 16 || m->d > 4096 || m->F <= 0 || m->F % 16 || m->V <= 0 || m->V % 16)
        return false;
    if (m->hidden3 != 3 * m->d) return false;
    if (m->Hq <= 0 || m->Hkv <= 0 || m->Hq % m->Hkv) return false;
    if (m->dh != 64 && m->dh != 128) return false;
    if (m->N < 1 || m->N > PD_MAX_LAYERS) return false;
    if (!(m->rms_eps > 0.f) || !(m->rope_theta > 0.f)) return false;
    if (!m->embed || !m->fc || !m->norm_emb || !m->norm_hid || !m->norm_final || !m->lm_head)
        return false;
    for (int l = 0; l < m->N; ++l) {
        if (!m->w_qkv[l] || !m->w_o[l] || !m->norm_post[l] || !m->w_gate[l] || !m->w_up[l] ||
            !m->w_down[l])
            return false;
        if (l > 0 && !m->norm_in[l]) return false;
    }
    return true;
}

bool batch_ok(const pd_batch* b, bool hidden_optional = false) {
    return b && b->input_ids && b->positions && b->slot_mapping && b->is_rejected &&
           b->is_masked && b->hidden_state_mapping && b->new_token_indices && b->cu_out &&
           b->seq_lens && (b->hidden || hidden_optional);
}

// Argument checks shared by the forward entry points (nothing is enqueued
// when they fail).
int forward_args_ok(const pd_model* m, const pd_batch_dims* dims, const pd_batch* b,
                    const int32_t* block_table, const uint16_t* kv_cache, const int32_t* draft_ids,
                    const pd_forward_opts* opts) {
    const uint16_t* hidden_d = opts ? opts->hidden_d : nullptr;
    const uint16_t* hidden_out = opts ? opts->hidden_out : nullptr;
    const bool fp8 = opts && opts->kv_fp8;
    const float* kv_scales = fp8 ? opts->kv_scales : nullptr;
    if (!model_ok(m) || !dims_ok(dims) || !batch_ok(b, hidden_d != nullptr)) return PD_EINVAL;
    if (kv_scales)
        for (int i = 0; i < 2 * m->N; ++i)
            if (!(kv_scales[i] > 0.f) || !std::isfinite(kv_scales[i])) return PD_EINVAL;
    if (((uintptr_t)hidden_d | (uintptr_t)hidden_out) & 15) return PD_EINVAL;
    if (dims->C == 0) return PD_OK;
    if (dims->block_size != PD_PAGE || dims->hidden3 != m->hidden3) return PD_EINVAL;
    if (!block_table || !kv_cache || !draft_ids) return PD_EINVAL;
    if (dims->max_blocks > PD_MAX_BLOCKS) return PD_EINVAL;
    if ((long long)dims->num_blocks * m->Hkv * PD_PAGE * m->dh * 2 * m->N > (1LL << 40))
        return PD_EINVAL;
    return PD_OK;
}

// The launch sequence of one drafter pass on scratch S (carved as L). h may
// be null (no event timing, no residual snapshots); st is the status word
// bad device data is reported to (may be null).
int forward_impl(pd_handle* h, char* S, const Layout& L, int32_t* st, const pd_model* m,
                 const pd_batch_dims* dims, const pd_batch* b, const int32_t* block_table,
                 uint16_t* kv_cache, int32_t* draft_ids, float* logits, const pd_forward_opts* opts,
                 hipStream_t s) {
    const uint16_t* hidden_d = opts ? opts->hidden_d : nullptr;
    uint16_t* hidden_out = opts ? opts->hidden_out : nullptr;
    const bool fp8 = opts && opts->kv_fp8;
    const float* kv_scales = fp8 ? opts->kv_scales : nullptr;
    int rc;
    float* x = (float*)(S + L.x);
    uint16_t* u = (uint16_t*)(S + L.u);
    uint16_t* q = (uint16_t*)(S + L.q);
    uint16_t* ao = (uint16_t*)(S + L.ao);
    uint16_t* act = (uint16_t*)(S + L.act);
    uint16_t* xg = (uint16_t*)(S + L.xg);
    float* ws = (float*)(S + L.ws);
    const int T = L.T, R = L.R, d = m->d;
    const int qkvw = (m->Hq + 2 * m->Hkv) * m->dh;
    const int hd = m->Hq * m->dh;
    // bytes of one K or V plane: bf16 elements or E4M3 codes
    const size_t plane = (size_t)dims->num_blocks * m->Hkv * PD_PAGE * m->dh * (fp8 ? 1 : 2);

    // one projection; returns its split count through *splits (EPI_PARTIAL)
    // compacted pass: the kept-row count and the split count of the latest
    // projection, both on the device
    int32_t* cnt = L.compact ? (int32_t*)(S + L.cnt) : nullptr;
    int32_t* t_dev = cnt;
    int32_t* s_dev = cnt ? cnt + 1 : nullptr;
    // one projection; returns its split count through *splits (EPI_PARTIAL;
    // with device row counts the most planes, the count itself in s_dev)
    auto gemm = [&](int cls, int epi, const uint16_t* X, int ldx, const int32_t* xrows,
                    int xlimit, const uint16_t* W, const uint16_t* W2, int M, int N, int K,
                    uint16_t* yb, int ldyb, int* splits, bool dev_rows = false) -> int {
        dev_rows = dev_rows && L.compact;
        GemmPlan p = plan_gemm(M, N, K, epi, dev_rows);
        if (splits) *splits = p.splits;
        GemmArgs a;
        std::memset(&a, 0, sizeof(a));
        if (dev_rows) {
            a.m_dev = t_dev;
            if (epi == EPI_PARTIAL) a.splits_out = s_dev;
        }
        a.X = X; a.ldx = ldx; a.xrows = xrows; a.xrows_limit = xlimit;
        a.W = W; a.W2 = W2; a.M = M; a.N = N; a.K = K;
        a.ws = ws; a.yb = yb; a.ldyb = ldyb;
        a.logits = logits; a.ldlog = m->V;
        a.amax_v = (float*)(S + L.amv); a.amax_i = (int*)(S + L.ami);
        a.status = st;
        Timed t(h, cls, s);
        return launch_gemm(epi, p, a, s);
    };
    // LM head on the packed sampled rows xg (one or two launches, see
    // plan_lm_head), argmax partials for all of V in every row
    auto lm_head = [&]() -> int {
        const LmHeadPlan lp = plan_lm_head(R, m->V, d);
        if (lp.ntiles != L.ntilesV) return PD_EINVAL;
        int r;
        for (int part = 0; part < 2; ++part) {
            const GemmPlan& p = part ? lp.tail : lp.main;
            if (p.kind < 0) break;
            const int n0 = part ? lp.n_main : 0;
            GemmArgs a;
            std::memset(&a, 0, sizeof(a));
            a.X = xg; a.ldx = d;
            a.W = m->lm_head + (size_t)n0 * d;
            a.M = R; a.N = part ? m->V - lp.n_main : lp.n_main; a.K = d;
            a.logits = logits ? logits + n0 : nullptr; a.ldlog = m->V;
            a.amax_v = (float*)(S + L.amv) + (part ? lp.main.ntiles : 0);
            a.amax_i = (int*)(S + L.ami) + (part ? lp.main.ntiles : 0);
            a.status = st;
            if (lp.tail.kind >= 0) {
                a.n_base = n0;
                a.amax_ld = lp.ntiles;
            }
            Timed t(h, PD_KERNEL_LMHEAD, s);
            if ((r = launch_gemm(EPI_ARGMAX, p, a, s)) != PD_OK) return r;
        }
        return PD_OK;
    };
    auto dbg = [&](int slot) -> int {
        if (!h || !h->dbg) return PD_OK;
        if (L.compact) {   // compacted rows back to their places (rejected rows are left as they are)
            Timed t(h, PD_KERNEL_OTHER, s);
            return launch_scatter_rows(x, h->dbg + (size_t)slot * T * d, (const int32_t*)(S + L.rowmap), t_dev,
                                       T, d, s);
        }
        return hipMemcpyAsync(h->dbg + (size_t)slot * T * d, x, (size_t)T * d * 4,
                              hipMemcpyDeviceToDevice, s) == hipSuccess ? PD_OK : PD_EHIP;
    };
#define PD_TRY(expr) do { if ((rc = (expr)) != PD_OK) return rc; } while (0)
    int sp = 1;
    // attention arguments shared by every layer; the split plan is built once
    AttnArgs aa;
    std::memset(&aa, 0, sizeof(aa));
    aa.positions = b->positions; aa.is_rejected = b->is_rejected;
    aa.cu_out = b->cu_out; aa.seq_lens = b->seq_lens; aa.block_table = block_table;
    aa.C = dims->C; aa.T = T; aa.Hq = m->Hq; aa.Hkv = m->Hkv;
    aa.max_blocks = dims->max_blocks; aa.num_blocks = dims->num_blocks;
    aa.sp = L.sp; aa.plan = (int32_t*)(S + L.plan);
    aa.scale_log2 = 1.4426950408889634f / sqrtf((float)m->dh);
    aa.part_o = (float*)(S + L.po); aa.part_ml = (float*)(S + L.pml);
    aa.out = ao; aa.status = st;

    if (L.dp.ok) {
        // the whole pass as one persistent launch (few rows: a chain of weight streams)
        DecodeArgs da;
        std::memset(&da, 0, sizeof(da));
        da.embed = m->embed; da.fc = m->fc; da.norm_emb = m->norm_emb; da.norm_hid = m->norm_hid;
        da.norm_final = m->norm_final; da.lm_head = m->lm_head;
        for (int l = 0; l < m->N; ++l) {
            da.norm_in[l] = m->norm_in[l]; da.w_qkv[l] = m->w_qkv[l]; da.w_o[l] = m->w_o[l];
            da.norm_post[l] = m->norm_post[l]; da.w_gate[l] = m->w_gate[l]; da.w_up[l] = m->w_up[l];
            da.w_down[l] = m->w_down[l];
        }
        da.d = d; da.Hq = m->Hq; da.Hkv = m->Hkv; da.dh = m->dh; da.F = m->F; da.NL = m->N; da.V = m->V;
        da.hidden3 = m->hidden3; da.eps = m->rms_eps;
        da.inv_step = std::pow((double)m->rope_theta, -2.0 / m->dh);
        da.ids = b->input_ids; da.positions = b->positions; da.slots = b->slot_mapping;
        da.new_idx = b->new_token_indices; da.hidden = b->hidden; da.hidden_d = hidden_d;
        da.hidden_out = hidden_out; da.T = T; da.R = R;
        da.kv = reinterpret_cast<char*>(kv_cache); da.plane_bytes = plane; da.num_blocks = dims->num_blocks;
        da.draft_ids = draft_ids; da.logits = logits;
        da.x = x; da.u = u; da.q = q; da.ao = ao; da.act = act; da.xg = xg; da.ws = ws;
        da.u_slot = (size_t)T * 2 * d;
        da.ao_slot = (size_t)T * hd;
        da.act_slot = (size_t)T * m->F;
        da.rows0 = L.dp.rows0;
        da.lm_in_kernel = L.dp.lm_in_kernel;
        da.amax_v = (float*)(S + L.amv); da.amax_i = (int*)(S + L.ami);
        da.dbg = h ? h->dbg : nullptr;
        da.timeline = h ? h->timeline : nullptr;
        da.sync = reinterpret_cast<unsigned*>(S + L.sync);
        da.status = st;
        da.sp_fc = L.dp.sp_fc; da.sp_qkv0 = L.dp.sp_qkv0; da.sp_qkv = L.dp.sp_qkv; da.sp_o = L.dp.sp_o;
        da.sp_down = L.dp.sp_down;
        da.g_fc = L.dp.g_fc; da.g_qkv0 = L.dp.g_qkv0; da.g_qkv = L.dp.g_qkv; da.g_o = L.dp.g_o;
        da.g_gu = L.dp.g_gu; da.g_down = L.dp.g_down; da.g_lm = L.dp.g_lm;
        da.at = aa;
        {
            Timed t(h, PD_KERNEL_DECODE, s);
            PD_TRY(launch_decode(L.dp, da, s));
        }
        if (L.dp.lm_in_kernel) return PD_OK;
        // LM head on the packed sampled rows the pass left in xg, greedy argmax
        PD_TRY(lm_head());
        Timed t(h, PD_KERNEL_OTHER, s);
        return launch_argmax_reduce((float*)(S + L.amv), (int*)(S + L.ami), R, L.ntilesV, draft_ids, st, s);
    }

    // Row compaction: the rows that are not rejected, in order, at the front
    // of every row buffer; the projections and row kernels stop at their
    // count (t_dev), attention sees the compacted request starts and no
    // rejected rows, and the LM head's sampled rows are renumbered.
    const uint16_t* hid = b->hidden;
    const int32_t* ids = b->input_ids;
    const int32_t* pos = b->positions;
    const int32_t* slots = b->slot_mapping;
    const int32_t* nti = b->new_token_indices;
    if (L.compact) {
        int32_t* cu_c = (int32_t*)(S + L.cu_c);
        int32_t* nti_c = (int32_t*)(S + L.nti_c);
        uint16_t* hid_c = (uint16_t*)(S + L.hid_c);
        int32_t* ids_c = (int32_t*)(S + L.ids_c);
        int32_t* pos_c = (int32_t*)(S + L.pos_c);
        int32_t* slot_c = (int32_t*)(S + L.slot_c);
        {
            Timed t(h, PD_KERNEL_OTHER, s);
            PD_TRY(launch_compact_rows(b->is_rejected, b->input_ids, b->positions, b->slot_mapping, b->cu_out,
                                       b->new_token_indices, b->hidden, T, dims->C, R, m->hidden3, hid_c, ids_c,
                                       pos_c, slot_c, cu_c, nti_c, (int32_t*)(S + L.rowmap), t_dev, st, s));
        }
        hid = hid_c; ids = ids_c; pos = pos_c; slots = slot_c; nti = nti_c;
        aa.positions = pos_c;
        aa.is_rejected = nullptr;
        aa.cu_out = cu_c;
    }
    // fc projection 3d -> d (starts the residual stream; skipped when the
    // projected rows are given), then the layer-0 input
    if (!hidden_d)
        PD_TRY(gemm(PD_KERNEL_GEMM, EPI_PARTIAL, hid, m->hidden3, nullptr, 0, m->fc, nullptr, T,
                    d, m->hidden3, nullptr, 0, &sp, true));
    {
        Timed t(h, PD_KERNEL_OTHER, s);
        // the attention split plan runs as one more workgroup of this launch
        PD_TRY(launch_layer0_input(hidden_d, ws, sp, ids, m->embed, m->V, x, m->norm_emb,
                                   m->norm_hid, u, T, d, m->rms_eps, st, s, &aa, t_dev, s_dev));
    }
    PD_TRY(dbg(0));
    for (int l = 0; l < m->N; ++l) {
        const int in_l = (l == 0) ? 2 * d : d;
        PD_TRY(gemm(PD_KERNEL_GEMM, EPI_PARTIAL, u, in_l, nullptr, 0, m->w_qkv[l], nullptr, T, qkvw,
                    in_l, nullptr, 0, &sp, true));
        char* kpl = reinterpret_cast<char*>(kv_cache) + (size_t)(2 * l) * plane;
        char* vpl = reinterpret_cast<char*>(kv_cache) + (size_t)(2 * l + 1) * plane;
        const float ks = kv_scales ? kv_scales[2 * l] : 1.0f, vs = kv_scales ? kv_scales[2 * l + 1] : 1.0f;
        {
            Timed t(h, PD_KERNEL_OTHER, s);
            PD_TRY(launch_rope_cache(ws, sp, pos, slots, T, m->Hq, m->Hkv, m->dh, m->rope_theta, q, kpl, vpl,
                                     dims->num_blocks, st, s, fp8 ? 1 : 0, ks, vs, t_dev, s_dev));
        }
        aa.q = q; aa.kplane = kpl; aa.vplane = vpl;
        aa.fp8 = fp8; aa.k_scale = ks; aa.v_scale = vs;
        {
            hipEvent_t e0 = nullptr, e1 = nullptr, e2 = nullptr, e3 = nullptr;
            if (h && (h->prof & (1 << PD_KERNEL_ATTN))) { e0 = take_event(h); e1 = take_event(h); }
            if (h && (h->prof & (1 << PD_KERNEL_OTHER))) { e2 = take_event(h); e3 = take_event(h); }
            rc = launch_attention(m->dh, aa, s, e0, e1, e2, e3);
            if (e0 && e1) h->ev[PD_KERNEL_ATTN].emplace_back(e0, e1);
            if (e2 && e3) h->ev[PD_KERNEL_OTHER].emplace_back(e2, e3);
            if (rc != PD_OK) return rc;
        }
        PD_TRY(gemm(PD_KERNEL_GEMM, EPI_PARTIAL, ao, hd, nullptr, 0, m->w_o[l], nullptr, T, d, hd,
                    nullptr, 0, &sp, true));
        {
            Timed t(h, PD_KERNEL_OTHER, s);
            PD_TRY(launch_resid_norm(ws, sp, x, m->norm_post[l], u, T, d, m->rms_eps, s, nullptr, 0, nullptr,
                                     nullptr, t_dev, s_dev));
        }
        PD_TRY(gemm(PD_KERNEL_GEMM, EPI_SWIGLU, u, d, nullptr, 0, m->w_gate[l], m->w_up[l], T, m->F,
                    d, act, m->F, nullptr, true));
        PD_TRY(gemm(PD_KERNEL_GEMM, EPI_PARTIAL, act, m->F, nullptr, 0, m->w_down[l], nullptr, T, d,
                    m->F, nullptr, 0, &sp, true));
        {
            Timed t(h, PD_KERNEL_OTHER, s);
            if (l + 1 < m->N) {
                // next layer's input norm
                PD_TRY(launch_resid_norm(ws, sp, x, m->norm_in[l + 1], u, T, d, m->rms_eps, s, nullptr, 0,
                                         nullptr, nullptr, t_dev, s_dev));
            } else if (h && h->dbg) {
                // the residual snapshot needs every row's final x
                PD_TRY(launch_resid_norm(ws, sp, x, m->norm_final, u, T, d, m->rms_eps, s, nullptr, 0, nullptr,
                                         nullptr, t_dev, s_dev));
            } else {
                // final norm of the K sampled rows of every request, packed for the LM head
                PD_TRY(launch_resid_norm(ws, sp, x, m->norm_final, xg, T, d, m->rms_eps, s, nti, R, st,
                                         hidden_out, nullptr, s_dev));
            }
        }
        PD_TRY(dbg(l + 1));
    }
    if (h && h->dbg) {
        Timed t(h, PD_KERNEL_OTHER, s);
        PD_TRY(launch_resid_norm(nullptr, 0, x, m->norm_final, xg, T, d, m->rms_eps, s, nti, R, st,
                                 hidden_out));
    }
    // LM head on the packed sampled rows, greedy argmax
    PD_TRY(lm_head());
    {
        Timed t(h, PD_KERNEL_OTHER, s);
        PD_TRY(launch_argmax_reduce((float*)(S + L.amv), (int*)(S + L.ami), R, L.ntilesV,
                                    draft_ids, st, s));
    }
#undef PD_TRY
    return PD_OK;
}


}  // namespace

extern "C" {

const char* pd_strerror(int code) {
    switch (code) {
        case PD_OK: return "ok";
        case PD_EINVAL: return "invalid argument";
        case PD_ENOMEM: return "device allocation failed";
        case PD_EHIP: return "HIP launch error";
        case PD_ESCRATCH: return "workspace exceeds the static scratch of the allocation-free forward";
        default: return "unknown error";
    }
}

int pd_expand_batch(const pd_batch_dims* dims, const pd_expand_in* in, const pd_batch* out,
                    void* stream) {
    if (!dims_ok(dims) || !in || !out) return PD_EINVAL;
    if (dims->C == 0) return PD_OK;
    if (!in->num_tokens || !in->num_rejected || !in->target_ids || !in->target_pos ||
        !in->target_hidden || !in->next_token_ids || !in->block_table || !in->h_shared)
        return PD_EINVAL;
    if (!batch_ok(out)) return PD_EINVAL;
    if (((uintptr_t)in->target_hidden | (uintptr_t)in->h_shared | (uintptr_t)out->hidden) & 15)
        return PD_EINVAL;
    return launch_expand(*dims, *in, *out, (hipStream_t)stream);
}

int pd_draft_forward(pd_handle** hp, const pd_model* m, const pd_batch_dims* dims,
                     const pd_batch* b, const int32_t* block_table, uint16_t* kv_cache,
                     int32_t* draft_ids, float* logits, void* stream) {
    return pd_draft_forward_ex(hp, m, dims, b, block_table, kv_cache, draft_ids, logits, nullptr,
                               stream);
}

int pd_draft_forward_ex(pd_handle** hp, const pd_model* m, const pd_batch_dims* dims,
                        const pd_batch* b, const int32_t* block_table, uint16_t* kv_cache,
                        int32_t* draft_ids, float* logits, const pd_forward_opts* opts,
                        void* stream) {
    if (!hp) return PD_EINVAL;
    int rc = forward_args_ok(m, dims, b, block_table, kv_cache, draft_ids, opts);
    if (rc != PD_OK || dims->C == 0) return rc;
    hipStream_t s = (hipStream_t)stream;
    if (!*hp) {
        if ((rc = create_handle(hp)) != PD_OK) return rc;
    }
    pd_handle* h = *hp;
    const Layout L = plan_layout(m, dims, opts && opts->kv_fp8, opts && opts->hidden_d);
    if ((rc = ensure_scratch(h, L.total, s)) != PD_OK) return rc;
    return forward_impl(h, h->scratch, L, h->status, m, dims, b, block_table, kv_cache, draft_ids, logits,
                        opts, s);
}

int pd_draft_forward_noalloc(const pd_model* m, const pd_batch_dims* dims, const pd_batch* b,
                             const int32_t* block_table, uint16_t* kv_cache, int32_t* draft_ids,
                             float* logits, const pd_forward_opts* opts, void* stream) {
    int rc = forward_args_ok(m, dims, b, block_table, kv_cache, draft_ids, opts);
    if (rc != PD_OK || dims->C == 0) return rc;
    const Layout L = plan_layout(m, dims, opts && opts->kv_fp8, opts && opts->hidden_d, kStaticScratchBytes);
    if (L.total > kStaticScratchBytes) return PD_ESCRATCH;
    char* S = nullptr;
    if ((rc = static_scratch(&S)) != PD_OK) return rc;
    return forward_impl(nullptr, S, L, b->status, m, dims, b, block_table, kv_cache, draft_ids, logits, opts,
                        (hipStream_t)stream);
}

int pd_ar_advance(const pd_batch_dims* dims_prev, const pd_batch* prev, const int32_t* draft_ids,
                  const int32_t* block_table, const pd_batch* next, void* stream) {
    if (!dims_ok(dims_prev) || !prev || !next || !draft_ids || !block_table) return PD_EINVAL;
    if (dims_prev->C == 0) return PD_OK;
    if (!prev->positions || !prev->new_token_indices) return PD_EINVAL;
    if (!next->input_ids || !next->positions || !next->slot_mapping || !next->is_rejected ||
        !next->is_masked || !next->hidden_state_mapping || !next->new_token_indices ||
        !next->cu_out || !next->seq_lens)
        return PD_EINVAL;
    return launch_ar_advance(*dims_prev, *prev, draft_ids, block_table, *next, (hipStream_t)stream);
}

int pd_verify_stub(const pd_batch_dims* dims_prev, const pd_batch* prev, const int32_t* prev_draft_ids,
                   const int32_t* prev_next_token_ids, const int32_t* accepted, int32_t* num_tokens,
                   int32_t* num_rejected, int32_t* target_ids, int32_t* target_pos, int32_t* status,
                   void* stream) {
    if (!dims_ok(dims_prev) || !prev) return PD_EINVAL;
    if (dims_prev->C == 0) return PD_OK;
    if (!prev->positions || !prev->new_token_indices || !prev_draft_ids || !prev_next_token_ids ||
        !accepted || !num_tokens || !num_rejected || !target_ids || !target_pos)
        return PD_EINVAL;
    return launch_verify_stub(*dims_prev, *prev, prev_draft_ids, prev_next_token_ids, accepted,
                              num_tokens, num_rejected, target_ids, target_pos, status,
                              (hipStream_t)stream);
}

int pd_seq_partition(const pd_partition_dims* dims, const uint8_t* keep, const int32_t* boundaries,
                     int32_t* seg, int32_t* seg_offsets, int32_t* rows, int32_t* status,
                     void* stream) {
    if (!dims) return PD_EINVAL;
    const pd_partition_dims& d = *dims;
    if (d.B < 0 || d.K < 1 || d.K > PD_PART_MAX_K || d.S < 1 || d.S > PD_PART_MAX_S || d.n < 8 ||
        d.n % 8 != 0 || (int64_t)d.K * ((d.n + 63) / 64) * 64 > PD_PART_MAX_POS)
        return PD_EINVAL;
    if (d.B == 0) return PD_OK;
    if (!keep || !boundaries || !seg || !seg_offsets || !rows) return PD_EINVAL;
    if (((uintptr_t)keep & 7) || ((uintptr_t)seg & 15) || ((uintptr_t)seg_offsets & 3) ||
        ((uintptr_t)rows & 3) || ((uintptr_t)boundaries & 3) || ((uintptr_t)status & 3))
        return PD_EINVAL;
    return launch_seq_partition(d, keep, boundaries, seg, seg_offsets, rows, status, (hipStream_t)stream);
}

void pd_free(pd_handle* h) {
    if (!h) return;
    (void)hipDeviceSynchronize();
    for (auto& v : h->ev)
        for (auto& p : v) {
            (void)hipEventDestroy(p.first);
            (void)hipEventDestroy(p.second);
        }
    for (auto e : h->spare) (void)hipEventDestroy(e);
    if (h->scratch) (void)hipFree(h->scratch);
    if (h->status) (void)hipFree(h->status);
    delete h;
}

int pd_status(pd_handle* h, int32_t* out, void* stream) {
    if (!h || !out) return PD_EINVAL;
    hipStream_t s = (hipStream_t)stream;
    if (hipStreamSynchronize(s) != hipSuccess) return PD_EHIP;
    if (hipMemcpy(out, h->status, sizeof(int32_t), hipMemcpyDeviceToHost) != hipSuccess)
        return PD_EHIP;
    if (hipMemset(h->status, 0, sizeof(int32_t)) != hipSuccess) return PD_EHIP;
    return hipDeviceSynchronize() == hipSuccess ? PD_OK : PD_EHIP;
}

int pd_set_debug_resid(pd_handle* h, float* dst) {
    if (!h) return PD_EINVAL;
    h->dbg = dst;
    return PD_OK;
}

int pd_set_decode_timeline(pd_handle* h, uint64_t* dst) {
    if (!h) return PD_EINVAL;
    h->timeline = dst;
    return PD_OK;
}

int pd_profile(pd_handle* h, int class_mask) {
    if (!h) return PD_EINVAL;
    (void)hipDeviceSynchronize();
    for (auto& v : h->ev) {
        for (auto& p : v) {
            h->spare.push_back(p.first);
            h->spare.push_back(p.second);
        }
        v.clear();
    }
    h->prof = class_mask & ((1 << PD_KERNEL_CLASSES) - 1);
    return PD_OK;
}

int pd_profile_read(pd_handle* h, int cls, double* total_ms, int64_t* launches) {
    if (!h || cls < 0 || cls >= PD_KERNEL_CLASSES || !total_ms || !launches) return PD_EINVAL;
    double tot = 0.0;
    for (auto& p : h->ev[cls]) {
        if (hipEventSynchronize(p.second) != hipSuccess) return PD_EHIP;
        float ms = 0.f;
        if (hipEventElapsedTime(&ms, p.first, p.second) != hipSuccess) return PD_EHIP;
        tot += ms;
    }
    *total_ms = tot;
    *launches = (int64_t)h->ev[cls].size();
    return PD_OK;
}

}  // extern "C"
