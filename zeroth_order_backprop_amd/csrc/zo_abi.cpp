// C ABI of the SPSA step: argument validation, the parameter arena layout,
// model dispatch and step sequencing.  Every check runs before the first
// launch, so a rejected call enqueues nothing.
//
// Step sequencing follows the ZOO blog ("Backprop 없이 Transformer를
// 학습시킨다"): two forwards per probe at +1 and -1 times the perturbation
// (section "zero-order optimization이란") inside the loop of the flowchart in
// section "backprop의 메모리 세금" (perturb, loss only, estimate, update).
#include <hip/hip_runtime.h>
#include <stdarg.h>
#include <stdio.h>
#include <string.h>

#include <algorithm>
#include <mutex>
#include <new>
#include <string>
#include <vector>

#include "zo_internal.hpp"
#include "zo_models.hpp"

namespace zo {

static thread_local char g_err[512] = "";

zo_status fail(zo_status st, const char* fmt, ...)
{
    va_list ap;
    va_start(ap, fmt);
    vsnprintf(g_err, sizeof g_err, fmt, ap);
    va_end(ap);
    return st;
}

zo_status check_launch(const char* what)
{
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return fail(ZO_ERR_HIP, "%s: %s", what, hipGetErrorString(e));
    return ZO_OK;
}

// ---------------------------------------------------------------- timing
namespace {
struct TimedLaunch {
    std::string family;
    hipEvent_t start, stop;
};
bool g_timing = false;
std::string g_timing_family;  // empty: every family
std::vector<TimedLaunch> g_timed;
std::vector<hipEvent_t> g_event_pool;

hipEvent_t take_event()
{
    if (!g_event_pool.empty()) {
        hipEvent_t e = g_event_pool.back();
        g_event_pool.pop_back();
        return e;
    }
    hipEvent_t e = nullptr;
    if (hipEventCreate(&e) != hipSuccess) return nullptr;
    return e;
}
}  // namespace

bool timing_active() { return g_timing; }

// A launch of family `have` belongs to the queried or selected family `want`
// when the two are equal or `have` is a sub-family "want.<name>".
static bool family_match(const std::string& have, const std::string& want)
{
    return have == want || (have.size() > want.size() && have.compare(0, want.size(), want) == 0 &&
                            have[want.size()] == '.');
}

KernelTimer::KernelTimer(const char* family, hipStream_t s) : slot_(-1), s_(s)
{
    if (!g_timing || (!g_timing_family.empty() && !family_match(family, g_timing_family))) return;
    TimedLaunch t{family, take_event(), take_event()};
    if (!t.start || !t.stop) return;
    (void)hipEventRecord(t.start, s);
    g_timed.push_back(t);
    slot_ = (int)g_timed.size() - 1;
}

KernelTimer::~KernelTimer()
{
    if (slot_ >= 0) (void)hipEventRecord(g_timed[slot_].stop, s_);
}

static uint64_t align64(uint64_t x) { return (x + 63) / 64 * 64; }

// Element count of every tensor of a model, in declaration order; returns the
// count (no allocation).  Tensor t of a decoder: 0 tok_emb, 1 pos_emb, then per
// layer ln1_g, ln1_b, w_qkv, w_o, ln2_g, ln2_b, w_up, w_down, then lnf_g, lnf_b.
static int tensor_sizes(const zo_model_desc* d, uint64_t* sizes, int cap)
{
    int n = 0;
    auto add = [&](uint64_t r, uint64_t c) {
        if (n < cap) sizes[n] = r * (c ? c : 1);
        ++n;
    };
    switch (d->kind) {
        case ZO_MODEL_LSQ:
            add(d->d_in, d->d_out);
            break;
        case ZO_MODEL_MLP:
            add(d->hidden, d->d_in);
            add(d->classes, d->hidden);
            break;
        case ZO_MODEL_DECODER: {
            const uint64_t D = d->d_model, F = d->ffn;
            add(d->vocab, D);
            add(d->max_seq, D);
            for (int64_t l = 0; l < d->layers; ++l) {
                add(D, 0); add(D, 0); add(3 * D, D); add(D, D);
                add(D, 0); add(D, 0); add(F, D); add(D, F);
            }
            add(D, 0);
            add(D, 0);
            break;
        }
    }
    return n;
}

// Arena offsets of the tensors (each at a multiple of 64 elements) and the
// arena length; `offs` holds kMaxTensors entries.  No allocation.
static int layout_offsets(const zo_model_desc* d, uint64_t* offs, uint64_t& total)
{
    const int n = tensor_sizes(d, offs, kMaxTensors);
    uint64_t off = 0;
    for (int t = 0; t < n && t < kMaxTensors; ++t) {
        off = align64(off);
        const uint64_t sz = offs[t];
        offs[t] = off;
        off += sz;
    }
    total = align64(off);
    return n;
}

// Tensors of a model in declaration order (the arena layout), with names.
static zo_status build_layout(const zo_model_desc* d, std::vector<zo_param_info>& out, uint64_t& total)
{
    uint64_t offs[kMaxTensors];
    const int n = layout_offsets(d, offs, total);
    if (n > kMaxTensors) return fail(ZO_ERR_UNSUPPORTED, "too many tensors");
    out.clear();
    auto add = [&](const std::string& name, int64_t r, int64_t c) {
        zo_param_info p;
        memset(&p, 0, sizeof p);
        snprintf(p.name, sizeof p.name, "%s", name.c_str());
        p.shape[0] = r;
        p.shape[1] = c;
        p.ndim = c > 0 ? 2 : 1;
        p.offset = offs[out.size()];
        out.push_back(p);
    };
    switch (d->kind) {
        case ZO_MODEL_LSQ:
            add("W", d->d_in, d->d_out);
            break;
        case ZO_MODEL_MLP:
            add("W1", d->hidden, d->d_in);
            add("W2", d->classes, d->hidden);
            break;
        case ZO_MODEL_DECODER: {
            const int64_t D = d->d_model;
            add("tok_emb", d->vocab, D);
            add("pos_emb", d->max_seq, D);
            for (int64_t l = 0; l < d->layers; ++l) {
                const std::string p = "l" + std::to_string(l) + ".";
                add(p + "ln1_g", D, 0);
                add(p + "ln1_b", D, 0);
                add(p + "w_qkv", 3 * D, D);
                add(p + "w_o", D, D);
                add(p + "ln2_g", D, 0);
                add(p + "ln2_b", D, 0);
                add(p + "w_up", d->ffn, D);
                add(p + "w_down", D, d->ffn);
            }
            add("lnf_g", D, 0);
            add("lnf_b", D, 0);
            break;
        }
        default:
            return fail(ZO_ERR_INVALID, "unknown model kind %d", d->kind);
    }
    return ZO_OK;
}

static zo_status validate_desc(const zo_model_desc* d)
{
    if (!d) return fail(ZO_ERR_INVALID, "null model description");
    if (d->batch <= 0) return fail(ZO_ERR_INVALID, "batch must be positive");
    switch (d->kind) {
        case ZO_MODEL_LSQ:
            if (d->dtype != ZO_F32) return fail(ZO_ERR_UNSUPPORTED, "least squares is fp32 only");
            if (d->d_in <= 0 || d->d_out <= 0) return fail(ZO_ERR_INVALID, "d_in, d_out must be positive");
            break;
        case ZO_MODEL_MLP:
            if (d->dtype != ZO_F32) return fail(ZO_ERR_UNSUPPORTED, "MLP is fp32 only");
            if (d->d_in <= 0 || d->hidden <= 0 || d->classes <= 0)
                return fail(ZO_ERR_INVALID, "d_in, hidden, classes must be positive");
            break;
        case ZO_MODEL_DECODER:
            if (d->dtype != ZO_BF16) return fail(ZO_ERR_UNSUPPORTED, "decoder is bf16 only");
            if (d->layers <= 0 || d->d_model <= 0 || d->heads <= 0 || d->ffn <= 0 || d->vocab <= 0 ||
                d->max_seq <= 0 || d->seq <= 0 || d->seq > d->max_seq)
                return fail(ZO_ERR_INVALID, "decoder sizes must be positive and seq <= max_seq");
            if (d->d_model % d->heads) return fail(ZO_ERR_INVALID, "d_model must divide into heads");
            if (d->layers > kMaxLayers) return fail(ZO_ERR_UNSUPPORTED, "at most %d layers", kMaxLayers);
            if (d->act != ZO_ACT_GELU && d->act != ZO_ACT_RELU) return fail(ZO_ERR_INVALID, "bad activation");
            break;
        default:
            return fail(ZO_ERR_INVALID, "unknown model kind %d", d->kind);
    }
    if (d->dirs != ZO_DIRS_GAUSS && d->dirs != ZO_DIRS_Q8) return fail(ZO_ERR_INVALID, "bad direction kind %d", d->dirs);
    return model_check_shape(*d);
}

// ------------------------------------------------- model-family dispatch
zo_status model_check_shape(const zo_model_desc& d)
{
    switch (d.kind) {
        case ZO_MODEL_LSQ: return lsq_check(d);
        case ZO_MODEL_MLP: return mlp_check(d);
        case ZO_MODEL_DECODER: return decoder_check(d);
    }
    return fail(ZO_ERR_INVALID, "unknown model kind");
}

size_t model_workspace_bytes(const zo_model_desc& d)
{
    switch (d.kind) {
        case ZO_MODEL_LSQ: return lsq_workspace(d);
        case ZO_MODEL_MLP: return mlp_workspace(d);
        case ZO_MODEL_DECODER: return decoder_workspace(d);
    }
    return 0;
}

zo_status model_forward(const ModelView& m, const zo_batch& b, const zo_pert* perts, int n_perts, double* loss,
                        hipStream_t s)
{
    switch (m.desc.kind) {
        case ZO_MODEL_LSQ: return lsq_forward(m, b, perts, n_perts, loss, s);
        case ZO_MODEL_MLP: return mlp_forward(m, b, perts, n_perts, loss, s);
        case ZO_MODEL_DECODER: return decoder_forward(m, b, perts, n_perts, loss, s);
    }
    return fail(ZO_ERR_INVALID, "unknown model kind");
}

static size_t dtype_size(int dtype) { return dtype == ZO_F32 ? 4 : 2; }

static bool overlap(const void* a, size_t na, const void* b, size_t nb)
{
    const char* pa = (const char*)a;
    const char* pb = (const char*)b;
    return pa < pb + nb && pb < pa + na;
}

// ---------------------------------------------- scratch of zo_step_noalloc
// Device memory for the workspace of zo_step_noalloc, for callers that cannot
// allocate: a file-scope array, one copy per GPU, held until the process ends.
// Host code never passes `scratch` itself (on the host that name is only a
// stand-in); it takes each device's address from hipGetSymbolAddress once,
// with that device current, and passes that pointer to the kernels.
constexpr size_t kScratchBytes = (size_t)64 << 20;
constexpr int kMaxDevices = 64;
static __device__ __align__(256) unsigned char scratch[kScratchBytes];

static std::mutex g_scratch_mu;
static void* g_scratch_ptr[kMaxDevices];

static zo_status scratch_of_current_device(void** out)
{
    int dev = -1;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0) return fail(ZO_ERR_HIP, "hipGetDevice failed");
    if (dev >= kMaxDevices) return fail(ZO_ERR_UNSUPPORTED, "device %d beyond the scratch table", dev);
    std::lock_guard<std::mutex> lock(g_scratch_mu);
    if (!g_scratch_ptr[dev]) {
        void* p = nullptr;
        const hipError_t e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
        if (e != hipSuccess || !p) return fail(ZO_ERR_HIP, "hipGetSymbolAddress(scratch): %s", hipGetErrorString(e));
        g_scratch_ptr[dev] = p;
    }
    *out = g_scratch_ptr[dev];
    return ZO_OK;
}

}  // namespace zo

using namespace zo;

struct zo_model {
    zo_model_desc desc;
    void* params;
    uint64_t n_params;
    void* workspace;
    size_t ws_bytes;
    std::vector<zo_param_info> layout;
    std::vector<uint64_t> offsets;
    void* graphs = nullptr;  // captured decoder forwards (decoder_graphs_free)
    void* copies = nullptr;  // the copies mode's arena copies + grouped workspace
    size_t copies_bytes = 0;
};

extern "C" {

const char* zo_status_str(zo_status st)
{
    switch (st) {
        case ZO_OK: return "ok";
        case ZO_ERR_INVALID: return "invalid argument";
        case ZO_ERR_UNSUPPORTED: return "unsupported dtype or shape";
        case ZO_ERR_HIP: return "HIP error";
        case ZO_ERR_NONFINITE: return "non-finite loss";
        case ZO_ERR_WORKSPACE: return "workspace too small";
    }
    return "unknown status";
}

const char* zo_last_error(void) { return g_err; }

zo_status zo_timing_enable(int32_t on)
{
    g_timing = on != 0;
    return ZO_OK;
}

zo_status zo_timing_select(const char* family)
{
    g_timing_family = family ? family : "";
    return ZO_OK;
}

zo_status zo_timing_reset(void)
{
    for (auto& t : g_timed) {
        g_event_pool.push_back(t.start);
        g_event_pool.push_back(t.stop);
    }
    g_timed.clear();
    return ZO_OK;
}

zo_status zo_timing_query(const char* family, double* total_ms, int64_t* launches)
{
    if (!family || !total_ms || !launches) return fail(ZO_ERR_INVALID, "null argument");
    double sum = 0.0;
    int64_t n = 0;
    const std::string want = family;
    for (auto& t : g_timed) {
        if (!family_match(t.family, want)) continue;
        if (hipEventSynchronize(t.stop) != hipSuccess) return fail(ZO_ERR_HIP, "event synchronise failed");
        float ms = 0.f;
        if (hipEventElapsedTime(&ms, t.start, t.stop) != hipSuccess) return fail(ZO_ERR_HIP, "event elapsed failed");
        sum += ms;
        ++n;
    }
    *total_ms = sum;
    *launches = n;
    return ZO_OK;
}

zo_status zo_param_layout(const zo_model_desc* desc, zo_param_info* out, int32_t cap, int32_t* n_out,
                          uint64_t* total)
{
    if (zo_status st = validate_desc(desc)) return st;
    if (!n_out || !total || (cap > 0 && !out)) return fail(ZO_ERR_INVALID, "null output pointer");
    std::vector<zo_param_info> v;
    uint64_t t = 0;
    if (zo_status st = build_layout(desc, v, t)) return st;
    for (int32_t k = 0; k < cap && k < (int32_t)v.size(); ++k) out[k] = v[k];
    *n_out = (int32_t)v.size();
    *total = t;
    return ZO_OK;
}

zo_status zo_workspace_bytes(const zo_model_desc* desc, size_t* bytes)
{
    if (zo_status st = validate_desc(desc)) return st;
    if (!bytes) return fail(ZO_ERR_INVALID, "null output pointer");
    *bytes = model_workspace_bytes(*desc);
    return ZO_OK;
}

zo_status zo_model_create(const zo_model_desc* desc, void* params, uint64_t n_params, void* workspace,
                          size_t ws_bytes, zo_model** out)
{
    if (zo_status st = validate_desc(desc)) return st;
    if (!out || !params) return fail(ZO_ERR_INVALID, "null params or output");
    std::vector<zo_param_info> v;
    uint64_t total = 0;
    if (zo_status st = build_layout(desc, v, total)) return st;
    if (n_params != total)
        return fail(ZO_ERR_INVALID, "arena has %llu elements, layout needs %llu", (unsigned long long)n_params,
                    (unsigned long long)total);
    if ((uintptr_t)params % 256 || (uintptr_t)workspace % 256)
        return fail(ZO_ERR_INVALID, "params and workspace must be 256-byte aligned");
    const size_t need = model_workspace_bytes(*desc);
    if (ws_bytes < need || (need && !workspace))
        return fail(ZO_ERR_WORKSPACE, "workspace %zu bytes, need %zu", ws_bytes, need);
    if (workspace && overlap(params, n_params * dtype_size(desc->dtype), workspace, ws_bytes))
        return fail(ZO_ERR_INVALID, "params and workspace overlap");
    zo_model* m = new (std::nothrow) zo_model;
    if (!m) return fail(ZO_ERR_INVALID, "out of host memory");
    m->desc = *desc;
    m->params = params;
    m->n_params = n_params;
    m->workspace = workspace;
    m->ws_bytes = ws_bytes;
    m->layout = v;
    for (const auto& p : v) m->offsets.push_back(p.offset);
    *out = m;
    return ZO_OK;
}

zo_status zo_model_destroy(zo_model* m)
{
    if (m) {
        decoder_graphs_free(m->graphs);
        if (m->copies) {
            (void)hipDeviceSynchronize();
            (void)hipFree(m->copies);
        }
    }
    delete m;
    return ZO_OK;
}

static ModelView view_of(zo_model* m)
{
    ModelView v;
    v.desc = m->desc;
    v.params = m->params;
    v.workspace = m->workspace;
    v.ws_bytes = m->ws_bytes;
    v.offsets = m->offsets.data();
    v.graphs = &m->graphs;
    v.copies = &m->copies;
    v.copies_bytes = &m->copies_bytes;
    return v;
}

zo_status zo_perturb(zo_model* m, uint64_t seed, uint32_t probe, float sigma, zo_stream s)
{
    if (!m) return fail(ZO_ERR_INVALID, "null model");
    return launch_perturb(m->params, m->desc.dtype, m->n_params, 0, seed, probe, sigma, (hipStream_t)s, m->desc.dirs);
}

static zo_status validate_batch(const zo_model_desc& d, const zo_batch* b)
{
    if (!b) return fail(ZO_ERR_INVALID, "null batch");
    if (b->batch <= 0 || b->batch > d.batch) return fail(ZO_ERR_INVALID, "batch size out of range");
    switch (d.kind) {
        case ZO_MODEL_LSQ:
            if (!b->x || !b->y) return fail(ZO_ERR_INVALID, "least squares needs x and y");
            break;
        case ZO_MODEL_MLP:
            if (!b->x || !b->labels) return fail(ZO_ERR_INVALID, "MLP needs x and labels");
            break;
        case ZO_MODEL_DECODER:
            if (!b->tokens) return fail(ZO_ERR_INVALID, "decoder needs tokens");
            if (b->seq < 2 || b->seq > d.seq) return fail(ZO_ERR_INVALID, "seq must be in 2..desc.seq");
            break;
    }
    // ids live in device memory and are not read here: an id out of range
    // makes the evaluation's loss NaN on the device instead
    if (((uintptr_t)b->labels | (uintptr_t)b->tokens) % 4)
        return fail(ZO_ERR_INVALID, "labels and tokens must be 4-byte aligned int32");
    if (((uintptr_t)b->x | (uintptr_t)b->y) % 4) return fail(ZO_ERR_INVALID, "x and y must be 4-byte aligned fp32");
    return ZO_OK;
}

zo_status zo_forward_loss(zo_model* m, const zo_batch* b, const zo_pert* perts, int32_t n_perts,
                          double* loss_dev, zo_stream s)
{
    if (!m || !loss_dev) return fail(ZO_ERR_INVALID, "null model or loss buffer");
    if (zo_status st = validate_batch(m->desc, b)) return st;
    if (n_perts < 0 || (n_perts > 0 && !perts)) return fail(ZO_ERR_INVALID, "bad perturbation list");
    if (n_perts > kMaxEvalsPerCall) return fail(ZO_ERR_INVALID, "at most %d perturbations per call", kMaxEvalsPerCall);
    if (n_perts > 0 && m->desc.dirs != ZO_DIRS_GAUSS && m->desc.kind != ZO_MODEL_DECODER)
        return fail(ZO_ERR_UNSUPPORTED, "perturbed evaluations with 8-bit directions are for decoders; use zo_perturb");
    return model_forward(view_of(m), *b, n_perts ? perts : nullptr, n_perts, loss_dev, (hipStream_t)s);
}

zo_status zo_update(zo_model* m, uint64_t seed, uint32_t n_probes, const double* g_dev, float lr, zo_stream s)
{
    if (!m || !g_dev) return fail(ZO_ERR_INVALID, "null model or g");
    if (n_probes == 0) return fail(ZO_ERR_INVALID, "n_probes must be >= 1");
    return launch_update(m->params, m->desc.dtype, m->n_params, 0, seed, n_probes, g_dev, lr, (hipStream_t)s,
                         m->desc.dirs);
}

static zo_status validate_step_cfg(const zo_model_desc& d, const zo_step_cfg* cfg)
{
    const uint32_t N = cfg->n_probes;
    if (N == 0 || N > 1024) return fail(ZO_ERR_INVALID, "n_probes must be in 1..1024");
    if (!(cfg->eps > 0.0f)) return fail(ZO_ERR_INVALID, "eps must be positive");
    if (cfg->mode != ZO_MODE_INPLACE && cfg->mode != ZO_MODE_FUSED && cfg->mode != ZO_MODE_COPIES)
        return fail(ZO_ERR_INVALID, "bad mode");
    if (cfg->precond != 0 && cfg->precond != 1) return fail(ZO_ERR_INVALID, "precond must be 0 or 1");
    if (cfg->precond && !(cfg->curv_floor > 0.0f)) return fail(ZO_ERR_INVALID, "curv_floor must be positive");
    if (cfg->mode == ZO_MODE_FUSED && d.dirs != ZO_DIRS_GAUSS && d.kind != ZO_MODEL_DECODER)
        return fail(ZO_ERR_UNSUPPORTED, "fused steps with 8-bit directions are for decoders; use the in-place mode");
    if (cfg->mode == ZO_MODE_COPIES && d.kind != ZO_MODEL_DECODER)
        return fail(ZO_ERR_UNSUPPORTED, "copies steps are for decoders");
    return ZO_OK;
}

// ---- the copies mode ----
// Evaluations at D(W +- eps z_i) materialised: 2P arena copies and the
// workspace of 2P evaluations side by side, in one device buffer owned by the
// model.  P: about kCopyRows token rows per forward, at most kMaxCopyProbes
// and N, the grouped activations under 2 GiB per buffer (the GEMMs' 32-bit
// offsets), and the buffer within half the free device memory.
constexpr int64_t kCopyRows = 131072;
constexpr uint32_t kMaxCopyProbes = 16;

static uint64_t copy_stride(uint64_t n_params) { return (n_params + 127) / 128 * 128; }

static uint32_t copies_probes(const zo_model_desc& d, uint32_t N, int64_t rows)
{
    int64_t p = rows % 256 ? 1 : std::max<int64_t>(1, (kCopyRows + 2 * rows - 1) / (2 * rows));
    p = std::min<int64_t>(p, std::min<uint32_t>(N, kMaxCopyProbes));
    const int64_t widest = std::max<int64_t>(3 * d.d_model, d.ffn);
    while (p > 1 && 2 * p * rows * widest * 2 >= (1ll << 31)) --p;
    return (uint32_t)p;
}

static size_t copies_bytes(const zo_model_desc& d, uint64_t n_params, uint32_t p)
{
    return 2 * p * copy_stride(n_params) * 2 + decoder_group_workspace(d, (int)(2 * p));
}

static zo_status copies_buffer(const ModelView& v, uint64_t n_params, uint32_t& p, void*& buf)
{
    if (!v.copies || !v.copies_bytes) return fail(ZO_ERR_UNSUPPORTED, "copies steps need zo_step (they allocate)");
    size_t need = copies_bytes(v.desc, n_params, p);
    if (*v.copies && *v.copies_bytes >= need) {
        buf = *v.copies;
        return ZO_OK;
    }
    if (*v.copies) {
        (void)hipDeviceSynchronize();
        (void)hipFree(*v.copies);
        *v.copies = nullptr;
        *v.copies_bytes = 0;
    }
    size_t free_b = 0, total_b = 0;
    if (hipMemGetInfo(&free_b, &total_b) != hipSuccess) return fail(ZO_ERR_HIP, "hipMemGetInfo failed");
    while (p > 1 && need > free_b / 2) need = copies_bytes(v.desc, n_params, --p);
    if (need > free_b) return fail(ZO_ERR_WORKSPACE, "copies steps need %zu bytes of device memory", need);
    if (hipMalloc(v.copies, need) != hipSuccess) {
        *v.copies = nullptr;
        return fail(ZO_ERR_WORKSPACE, "cannot allocate %zu bytes for the copies step", need);
    }
    *v.copies_bytes = need;
    buf = *v.copies;
    return ZO_OK;
}

// The step's launches, after validation (shared by zo_step and
// zo_step_noalloc; allocates nothing).
static zo_status run_step(const ModelView& v, uint64_t n_params, const zo_batch& b, const zo_step_cfg& cfg,
                          double* losses_dev, double* g_dev, hipStream_t st)
{
    const zo_model_desc& d = v.desc;
    const uint32_t N = cfg.n_probes;
    const float sig = cfg.eps;
    const float sig2 = -2.0f * cfg.eps;
    // 1.5-SPSA: the clean evaluation at the stored weights, before any probe
    if (cfg.precond)
        if (zo_status r = model_forward(v, b, nullptr, 0, losses_dev + 2 * N, st)) return r;
    if (cfg.mode == ZO_MODE_INPLACE) {
        for (uint32_t i = 0; i < N; ++i) {
            zo_status r = launch_perturb(v.params, d.dtype, n_params, 0, cfg.seed, i, sig, st, d.dirs);
            if (r) return r;
            zo_status f1 = model_forward(v, b, nullptr, 0, losses_dev + 2 * i, st);
            // the restore sequence always completes once a probe has started
            zo_status r2 = launch_perturb(v.params, d.dtype, n_params, 0, cfg.seed, i, sig2, st, d.dirs);
            zo_status f2 = f1 ? f1 : model_forward(v, b, nullptr, 0, losses_dev + 2 * i + 1, st);
            // the last probe's restore is applied together with the update below
            const bool defer = i + 1 == N && !f1 && !r2 && !f2;
            zo_status r3 = defer ? ZO_OK : launch_perturb(v.params, d.dtype, n_params, 0, cfg.seed, i, sig, st, d.dirs);
            if (f1) return f1;
            if (r2) return r2;
            if (f2) return f2;
            if (r3) return r3;
        }
    } else if (cfg.mode == ZO_MODE_COPIES) {
        uint32_t P = copies_probes(d, N, (int64_t)d.batch * d.seq);
        void* buf = nullptr;
        if (zo_status r = copies_buffer(v, n_params, P, buf)) return r;
        // layout: 2P copies of cs elements, then the workspace of 2P evaluations
        const uint64_t cs = copy_stride(n_params);
        void* ws = (char*)buf + 2 * (size_t)P * cs * 2;
        const bool side_by_side = (int64_t)b.batch * b.seq % 256 == 0;
        for (uint32_t k = 0; k < N; k += P) {
            const uint32_t np = std::min(P, N - k);
            if (zo_status r = launch_perturb_copies(v.params, buf, cs, n_params, cfg.seed, k, np, sig, st, d.dirs))
                return r;
            if (side_by_side) {
                if (zo_status r = decoder_forward_groups(v, b, buf, (int)(2 * np), cs, ws, losses_dev + 2 * k, st))
                    return r;
                continue;
            }
            for (uint32_t c = 0; c < 2 * np; ++c)
                if (zo_status r = decoder_forward_groups(v, b, (const uint16_t*)buf + c * cs, 1, 0, ws,
                                                         losses_dev + 2 * k + c, st))
                    return r;
        }
    } else {
        // evaluations (L+_0, L-_0, L+_1, ...) in launches of at most kMaxEvalsPerCall
        zo_pert perts[kMaxEvalsPerCall];
        for (uint32_t k = 0; k < 2 * N; k += kMaxEvalsPerCall) {
            const int32_t cnt = (int32_t)std::min<uint32_t>(kMaxEvalsPerCall, 2 * N - k);
            for (int32_t e = 0; e < cnt; ++e) {
                const uint32_t q = k + (uint32_t)e;
                perts[e] = zo_pert{cfg.seed, q / 2, (q & 1) ? -sig : sig};
            }
            if (zo_status r = model_forward(v, b, perts, cnt, losses_dev + k, st)) return r;
        }
    }
    zo_status r = cfg.precond ? launch_precond(losses_dev, N, cfg.eps, cfg.curv_floor, g_dev, st)
                              : launch_gscalar(losses_dev, N, cfg.eps, g_dev, st);
    if (cfg.mode == ZO_MODE_INPLACE) {
        // the last probe's restore (+eps) and the update, in one pass; the
        // restore is written even if the scalars could not be formed
        if (r) {
            launch_perturb(v.params, d.dtype, n_params, 0, cfg.seed, N - 1, sig, st, d.dirs);
            return r;
        }
        return launch_restore_update(v.params, d.dtype, n_params, cfg.seed, N, g_dev, cfg.lr, sig, st, d.dirs);
    }
    if (r) return r;
    return launch_update(v.params, d.dtype, n_params, 0, cfg.seed, N, g_dev, cfg.lr, st, d.dirs);
}

zo_status zo_step(zo_model* m, const zo_batch* b, const zo_step_cfg* cfg, double* losses_dev, double* g_dev,
                  zo_stream s)
{
    if (!m || !cfg || !losses_dev || !g_dev) return fail(ZO_ERR_INVALID, "null argument");
    if (zo_status st = validate_batch(m->desc, b)) return st;
    if (zo_status st = validate_step_cfg(m->desc, cfg)) return st;
    return run_step(view_of(m), m->n_params, *b, *cfg, losses_dev, g_dev, (hipStream_t)s);
}

zo_status zo_step_noalloc(const zo_model_desc* desc, void* params, uint64_t n_params, const zo_batch* b,
                          const zo_step_cfg* cfg, double* losses_dev, double* g_dev, zo_stream s)
{
    if (!desc || !params || !cfg || !losses_dev || !g_dev) return fail(ZO_ERR_INVALID, "null argument");
    if (zo_status st = validate_desc(desc)) return st;
    uint64_t offs[kMaxTensors];
    uint64_t total = 0;
    if (layout_offsets(desc, offs, total) > kMaxTensors) return fail(ZO_ERR_UNSUPPORTED, "too many tensors");
    if (n_params != total)
        return fail(ZO_ERR_INVALID, "arena has %llu elements, layout needs %llu", (unsigned long long)n_params,
                    (unsigned long long)total);
    if ((uintptr_t)params % 256) return fail(ZO_ERR_INVALID, "params must be 256-byte aligned");
    const size_t need = model_workspace_bytes(*desc);
    if (need > kScratchBytes)
        return fail(ZO_ERR_WORKSPACE, "this model needs %zu bytes of scratch; zo_step_noalloc holds %zu", need,
                    (size_t)kScratchBytes);
    if (zo_status st = validate_batch(*desc, b)) return st;
    if (zo_status st = validate_step_cfg(*desc, cfg)) return st;
    if (cfg->mode == ZO_MODE_COPIES) return fail(ZO_ERR_UNSUPPORTED, "copies steps allocate; use zo_step");
    void* scratch_dev = nullptr;
    if (zo_status st = scratch_of_current_device(&scratch_dev)) return st;
    if (overlap(params, n_params * dtype_size(desc->dtype), scratch_dev, kScratchBytes))
        return fail(ZO_ERR_INVALID, "params overlap the library's scratch");
    ModelView v;
    v.desc = *desc;
    v.params = params;
    v.workspace = scratch_dev;
    v.ws_bytes = kScratchBytes;
    v.offsets = offs;
    return run_step(v, n_params, *b, *cfg, losses_dev, g_dev, (hipStream_t)s);
}

zo_status zo_step_split(zo_model* m, const zo_batch* b, const zo_split_cfg* cfg, double* losses_dev,
                        double* g1_dev, double* g2_dev, zo_stream s)
{
    if (!m || !cfg || !losses_dev || !g1_dev || !g2_dev) return fail(ZO_ERR_INVALID, "null argument");
    if (zo_status st = validate_batch(m->desc, b)) return st;
    if (!(cfg->eps > 0.0f)) return fail(ZO_ERR_INVALID, "eps must be positive");
    if (m->desc.dirs != ZO_DIRS_GAUSS) return fail(ZO_ERR_UNSUPPORTED, "split perturbation uses Gaussian directions");
    if (zo_status st = mlp_split_check(m->desc, (int)cfg->p1, (int)cfg->ps)) return st;
    return mlp_split_step(view_of(m), *b, cfg->seed, (int)cfg->p1, (int)cfg->ps, cfg->eps, cfg->lr, losses_dev,
                          g1_dev, g2_dev, (hipStream_t)s);
}

zo_status zo_step_dust(zo_model* m, const zo_batch* b, const zo_dust_cfg* cfg, double* losses_dev, zo_stream s)
{
    if (!m || !cfg || !losses_dev) return fail(ZO_ERR_INVALID, "null argument");
    if (zo_status st = validate_batch(m->desc, b)) return st;
    if (!(cfg->sigma1 > 0.0f) || !(cfg->sigma2 > 0.0f)) return fail(ZO_ERR_INVALID, "sigma1, sigma2 must be positive");
    if (zo_status st = mlp_dust_check(m->desc, *b, (int)cfg->k1, (int)cfg->k2)) return st;
    return mlp_dust_step(view_of(m), *b, cfg->seed, (int)cfg->k1, (int)cfg->k2, cfg->sigma1, cfg->sigma2, cfg->lr,
                         losses_dev, (hipStream_t)s);
}

zo_status zo_replay_step(zo_model* m, const zo_step_cfg* cfg, const double* g_dev, zo_stream s)
{
    if (!m || !cfg || !g_dev) return fail(ZO_ERR_INVALID, "null argument");
    const uint32_t N = cfg->n_probes;
    if (N == 0 || N > 1024) return fail(ZO_ERR_INVALID, "n_probes must be in 1..1024");
    if (!(cfg->eps > 0.0f)) return fail(ZO_ERR_INVALID, "eps must be positive");
    if (cfg->mode != ZO_MODE_INPLACE && cfg->mode != ZO_MODE_FUSED && cfg->mode != ZO_MODE_COPIES)
        return fail(ZO_ERR_INVALID, "bad mode");
    hipStream_t st = (hipStream_t)s;
    if (cfg->mode == ZO_MODE_INPLACE) {
        // the step's perturb / restore passes, in its order, without the evaluations
        const float sig = cfg->eps, sig2 = -2.0f * cfg->eps;
        for (uint32_t i = 0; i < N; ++i)
            for (float sg : {sig, sig2, sig})
                if (zo_status r = launch_perturb(m->params, m->desc.dtype, m->n_params, 0, cfg->seed, i, sg, st, m->desc.dirs))
                    return r;
    }
    return launch_update(m->params, m->desc.dtype, m->n_params, 0, cfg->seed, N, g_dev, cfg->lr, st, m->desc.dirs);
}

static zo_status check_buffer(const void* w, int32_t dtype, int32_t dirs, uint64_t j0)
{
    if (!w) return fail(ZO_ERR_INVALID, "null buffer");
    if (dtype != ZO_F32 && dtype != ZO_BF16) return fail(ZO_ERR_UNSUPPORTED, "dtype must be F32 or BF16");
    if (dirs != ZO_DIRS_GAUSS && dirs != ZO_DIRS_Q8) return fail(ZO_ERR_INVALID, "bad direction kind %d", dirs);
    if ((uintptr_t)w % 16) return fail(ZO_ERR_INVALID, "buffer must be 16-byte aligned");
    if (j0 % (dirs == ZO_DIRS_Q8 ? 16 : 4)) return fail(ZO_ERR_INVALID, "j0 must be a multiple of 4 (16 for 8-bit)");
    return ZO_OK;
}

zo_status zo_perturb_buffer(void* w, int32_t dtype, int32_t dirs, uint64_t n, uint64_t j0, uint64_t seed,
                            uint32_t probe, float sigma, zo_stream s)
{
    if (zo_status st = check_buffer(w, dtype, dirs, j0)) return st;
    if (n == 0) return ZO_OK;
    return launch_perturb(w, dtype, n, j0, seed, probe, sigma, (hipStream_t)s, dirs);
}

zo_status zo_update_buffer(void* w, int32_t dtype, int32_t dirs, uint64_t n, uint64_t j0, uint64_t seed,
                           uint32_t n_probes, const double* g_dev, float lr, zo_stream s)
{
    if (zo_status st = check_buffer(w, dtype, dirs, j0)) return st;
    if (!g_dev) return fail(ZO_ERR_INVALID, "null g");
    if (n_probes == 0) return fail(ZO_ERR_INVALID, "n_probes must be >= 1");
    if (n == 0) return ZO_OK;
    return launch_update(w, dtype, n, j0, seed, n_probes, g_dev, lr, (hipStream_t)s, dirs);
}

zo_status zo_gscalar(const double* losses_dev, uint32_t n, float eps, double* g_dev, zo_stream s)
{
    if (!losses_dev || !g_dev) return fail(ZO_ERR_INVALID, "null argument");
    if (n == 0) return ZO_OK;
    return launch_gscalar(losses_dev, n, eps, g_dev, (hipStream_t)s);
}

zo_status zo_debug_rng(uint64_t seed, uint32_t probe, uint64_t j0, uint64_t n, uint32_t* words_dev, float* z_dev,
                       zo_stream s)
{
    if (!words_dev && !z_dev) return fail(ZO_ERR_INVALID, "both outputs null");
    return launch_debug_rng(seed, probe, j0, n, words_dev, z_dev, (hipStream_t)s);
}

zo_status zo_debug_box_muller(const uint32_t* pairs_dev, uint64_t n_pairs, float* z_dev, zo_stream s)
{
    if (!pairs_dev || !z_dev) return fail(ZO_ERR_INVALID, "null argument");
    return launch_debug_box_muller(pairs_dev, n_pairs, z_dev, (hipStream_t)s);
}

zo_status zo_debug_gemm_bf16(const void* A_dev, const void* W_dev, void* C_dev, int32_t M, int32_t N, int32_t K,
                             int32_t epi, zo_stream s)
{
    return debug_gemm_bf16(A_dev, W_dev, C_dev, M, N, K, epi, (hipStream_t)s);
}

zo_status zo_debug_attention(const void* qkv_dev, void* out_dev, int32_t B, int32_t S, int32_t H, int32_t dh,
                             zo_stream s)
{
    return debug_attention(qkv_dev, out_dev, B, S, H, dh, (hipStream_t)s);
}

zo_status zo_debug_layernorm(const void* h_dev, const void* g_dev, const void* b_dev, void* x_dev, int32_t rows,
                             int32_t d, zo_stream s)
{
    return debug_layernorm(h_dev, g_dev, b_dev, x_dev, rows, d, (hipStream_t)s);
}

}  // extern "C"
