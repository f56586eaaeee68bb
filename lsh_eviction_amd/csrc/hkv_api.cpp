// hkv_api.cpp -- the C ABI of libhkv.so: handle, validation before any
// enqueue, workspace carving, launch sequencing, checkpoint and introspection.
#include <hip/hip_runtime.h>

#include <cstdio>
#include <cstdlib>
#include <cstring>
#include <mutex>
#include <string>
#include <vector>

#include "hkv.h"
#include "hkv_kernels.h"
#include "hkv_layout.h"

struct hkv_cache {
    hkv::Layout lay;
    hkv::DevCache dev;
    std::vector<int32_t> budgets;
    std::vector<int32_t> plens;
    int device = 0;
    int last_n_max = 0;
    bool prefilled = false;
    bool last_query_prefill = false;
    bool stepped = false;
    bool obs_codes = false;    // dbg_q holds a CHUNK prefill's observation codes
    bool poisoned = false;
    bool debug_sync = false;
    bool debug_nan = false;    // HKV_DEBUG_NAN=1: partial results poisoned with NaN before each step
    std::string err;
};

namespace {

thread_local std::string g_err;

hkv_status fail(hkv_cache* c, hkv_status s, const std::string& msg)
{
    if (c)
        c->err = msg;
    else
        g_err = msg;
    return s;
}

bool aligned(const void* p, size_t a) { return ((uintptr_t)p % a) == 0; }

// Checks a launch; a failure poisons the handle.
hkv_status check_launch(hkv_cache* c, hipError_t e, hipStream_t st, const char* what)
{
    if (e == hipSuccess && c->debug_sync) e = hipStreamSynchronize(st);
    if (e == hipSuccess && c->debug_sync) e = hipGetLastError();
    if (e != hipSuccess) {
        c->poisoned = true;
        return fail(c, HKV_ERR_DEVICE, std::string(what) + ": " + hipGetErrorString(e));
    }
    return HKV_OK;
}

hkv_status usable(hkv_cache* c)
{
    if (!c) return HKV_ERR_INVALID_ARG;
    if (c->poisoned) return fail(c, HKV_ERR_STATE, "handle poisoned by an earlier device error");
    return HKV_OK;
}

}  // namespace

extern "C" const char* hkv_last_error(const hkv_cache* c) { return c ? c->err.c_str() : g_err.c_str(); }

// ---------------------------------------------------------------------------
// Per-step scratch of hkv_decode_step_static, for callers that cannot
// allocate: a file-scope device array, one copy per GPU, alive until the
// process ends.  Host code never passes the array's name to a kernel (on the
// host it is a stand-in, not a device address): hkv_create resolves its
// device address once per device, with that device current, and the entry
// point uses only that address.
// ---------------------------------------------------------------------------
namespace {

constexpr size_t kStaticScratchBytes = 8u << 20;
constexpr int kMaxDevices = 64;

static __device__ __align__(256) unsigned char scratch[kStaticScratchBytes];

std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices] = {};

// Device address of `scratch` on the current device `dev` (resolved once).
hipError_t resolve_static_scratch(int dev)
{
    if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
    std::lock_guard<std::mutex> lk(g_scratch_mu);
    if (g_scratch_ptr[dev]) return hipSuccess;
    void* p = nullptr;
    hipError_t e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return e;
    if (!p) return hipErrorInvalidSymbol;
    g_scratch_ptr[dev] = p;
    return hipSuccess;
}

void* static_scratch(int dev)
{
    if (dev < 0 || dev >= kMaxDevices) return nullptr;
    std::lock_guard<std::mutex> lk(g_scratch_mu);
    return g_scratch_ptr[dev];
}

// The per-step scratch of a decode step carved from `base` (256-byte
// aligned pieces, as in the workspace): the fused step's records, candidate
// rows, eviction keys and ticket counters, and the split schedule's
// partials.  Returns the bytes used.
size_t carve_step_scratch(const hkv::Layout& L, char* base, hkv::DevCache* d)
{
    const size_t heads = (size_t)L.B * L.Hkv;
    size_t off = 0;
    auto take = [&](size_t bytes) {
        const size_t o = off;
        off = (off + bytes + hkv::kAlign - 1) / hkv::kAlign * hkv::kAlign;
        return o;
    };
    const size_t frec = take(heads * L.nsplit * L.G * L.d * 4);
    const size_t fscal = take(heads * L.nsplit * L.G * 16);
    const size_t cand_v = take(heads * L.nsplit * L.d * 4);
    const size_t part = take((size_t)L.B * L.Hq * L.nsplit * (L.d + 4) * 4);
    const size_t ekey = take(heads * 2 * 8);
    const size_t count = take(heads * hkv::kCountStride * 4);
    if (d && base) {
        d->frec = (float*)(base + frec);
        d->fscal = (float*)(base + fscal);
        d->cand_v = (float*)(base + cand_v);
        d->part = (float*)(base + part);
        d->ekey = (unsigned long long*)(base + ekey);
        d->count = (unsigned*)(base + count);
    }
    return off;
}

}  // namespace

extern "C" hkv_status hkv_create(const hkv_config* cfg, const float* R_host, void* workspace,
                                 size_t ws_bytes, void* stream, hkv_cache** out)
{
    char msg[256] = {0};
    if (!out) return fail(nullptr, HKV_ERR_INVALID_ARG, "out is NULL");
    *out = nullptr;
    hkv::Layout L;
    hkv_status s = hkv::compute_layout(cfg, &L, msg, sizeof(msg));
    if (s != HKV_OK) return fail(nullptr, s, msg);
    if (!R_host) return fail(nullptr, HKV_ERR_INVALID_ARG, "R is NULL");
    if (!workspace) return fail(nullptr, HKV_ERR_INVALID_ARG, "workspace is NULL");
    if (!aligned(workspace, hkv::kAlign)) return fail(nullptr, HKV_ERR_INVALID_ARG, "workspace not 256-byte aligned");
    if (ws_bytes < L.total) {
        snprintf(msg, sizeof(msg), "workspace has %zu bytes, %zu needed", ws_bytes, L.total);
        return fail(nullptr, HKV_ERR_INVALID_ARG, msg);
    }
    hipStream_t st = (hipStream_t)stream;
    int dev = 0;
    hipError_t ge = hipGetDevice(&dev);
    if (ge == hipSuccess) ge = resolve_static_scratch(dev);
    if (ge != hipSuccess) {
        (void)hipGetLastError();
        return fail(nullptr, HKV_ERR_DEVICE, std::string("hkv_create: device address of the static scratch: ") +
                                                 hipGetErrorString(ge));
    }
    hkv_cache* c = new hkv_cache();
    c->lay = L;
    c->budgets.assign(cfg->budgets, cfg->budgets + cfg->batch);
    c->plens.assign(cfg->batch, 0);
    const char* dbg = getenv("HKV_DEBUG");
    c->debug_sync = dbg && dbg[0] == '1';
    const char* dnan = getenv("HKV_DEBUG_NAN");
    c->debug_nan = dnan && dnan[0] == '1';
    if (hipGetDevice(&c->device) != hipSuccess) c->device = 0;

    char* ws = (char*)workspace;
    hkv::DevCache& d = c->dev;
    d.R = (const float*)(ws + L.off_R);
    d.budget = (const int*)(ws + L.off_budget);
    d.plen = (const int*)(ws + L.off_plen);
    d.state = (int*)(ws + L.off_state);
    d.K = ws + L.off_K;
    d.V = ws + L.off_V;
    d.code = ws + L.off_code;
    d.tok = (int*)(ws + L.off_tok);
    d.dbg_q = (uint32_t*)(ws + L.off_dbg_q);
    d.dbg_k = (uint32_t*)(ws + L.off_dbg_k);
    d.part = (float*)(ws + L.off_part);
    d.frec = (float*)(ws + L.off_frec);
    d.fscal = (float*)(ws + L.off_fscal);
    d.cand_v = (float*)(ws + L.off_cand_v);
    d.ekey = (unsigned long long*)(ws + L.off_ekey);
    d.info = (int*)(ws + L.off_info);
    d.count = (unsigned*)(ws + L.off_count);
    d.pcode = ws + L.off_pcode;
    d.qcode = ws + L.off_qcode;
    d.vs = (float*)(ws + L.off_vs);
    d.vbits = L.value_bits;
    d.B = L.B; d.Hq = L.Hq; d.Hkv = L.Hkv; d.G = L.G; d.d = L.d; d.bits = L.bits; d.W = L.W;
    d.Smax = L.Smax; d.chunk = L.chunk; d.nsplit = L.nsplit;
    d.ragged = L.nblk > 0;
    d.blk = (const uint2*)(ws + L.off_blk);
    d.nblk = L.nblk;
    d.kv_bf16 = L.kv_dtype == HKV_BF16;
    d.code_slots = (long long)L.code_slots;
    d.pcode_slots = (long long)L.pcode_slots;
    d.csum = (int*)(ws + L.off_csum);
    d.pchunk = L.pchunk;
    d.nchunk_max = (long long)L.nchunk_max;
    d.chist = (int*)(ws + L.off_chist);
    d.chist_bins = L.chist_bins;
    d.tK = d.tV = nullptr;
    d.ttok = nullptr;
    d.tcount = L.tcap > 0 ? (int*)(ws + L.off_tcount) : nullptr;
    d.tpart = L.tcap > 0 ? (float*)(ws + L.off_tpart) : nullptr;
    d.tflag = L.tcap > 0 ? (unsigned*)(ws + L.off_tflag) : nullptr;
    d.tcap = L.tcap;
    d.tsplit = L.tsplit;
    d.tflag_words = (long long)L.tflag_words;

    hipError_t e = hipMemcpyAsync((void*)d.R, R_host, (size_t)L.d * L.bits * sizeof(float),
                                  hipMemcpyHostToDevice, st);
    if (e == hipSuccess)
        e = hipMemcpyAsync((void*)d.budget, cfg->budgets, (size_t)L.B * sizeof(int32_t),
                           hipMemcpyHostToDevice, st);
    if (e == hipSuccess && L.nblk > 0) {
        std::vector<uint32_t> blk((size_t)L.nblk * 2);
        hkv::fused_block_order(cfg->budgets, cfg->batch, L.chunk, blk.data());
        e = hipMemcpy((void*)d.blk, blk.data(), blk.size() * 4, hipMemcpyHostToDevice);
    }
    if (e == hipSuccess) e = hkv::launch_reset(d, st);
    // value scales start at zero (the attention tile reads the scales of 16 rows at once)
    if (e == hipSuccess && L.value_bits != 0)
        e = hipMemsetAsync(d.vs, 0, ((size_t)L.B * L.Hkv * L.Smax + 16) * 4, st);
    if (e == hipSuccess) e = hipStreamSynchronize(st);
    if (e != hipSuccess) {
        std::string m = std::string("hkv_create: ") + hipGetErrorString(e);
        delete c;
        return fail(nullptr, HKV_ERR_DEVICE, m);
    }
    *out = c;
    return HKV_OK;
}

extern "C" hkv_status hkv_destroy(hkv_cache* c)
{
    if (!c) return HKV_ERR_INVALID_ARG;
    delete c;
    return HKV_OK;
}

// Entries per head of a kept-chunk list: ceil(Smax / C).
static int chunk_list_len(const hkv::Layout& L) { return L.pchunk ? (L.Smax + L.pchunk - 1) / L.pchunk : 0; }

// Checks shared by the prefill calls, then the prompt lengths go to the
// device and the kernels are enqueued.
static hkv_status prefill_impl(hkv_cache* c, const void* K, const void* V, const float* Q,
                               const int32_t* prompt_lens, int32_t n_max, void* stream, const char* fn,
                               const int32_t* reuse = nullptr, int32_t* kept = nullptr)
{
    const std::string f(fn);
    if (c->prefilled) return fail(c, HKV_ERR_STATE, f + ": cache is not empty");
    if (!prompt_lens) return fail(c, HKV_ERR_INVALID_ARG, f + ": prompt_lens is NULL");
    if (n_max < 0 || n_max > c->lay.max_prompt)
        return fail(c, HKV_ERR_INVALID_ARG,
                    f + ": n_max " + std::to_string(n_max) + " outside [0, max_prompt = " +
                        std::to_string(c->lay.max_prompt) + "]");
    for (int b = 0; b < c->lay.B; ++b)
        if (prompt_lens[b] < 0 || prompt_lens[b] > n_max)
            return fail(c, HKV_ERR_INVALID_ARG,
                        f + ": prompt_lens[" + std::to_string(b) + "] outside [0, n_max]");
    if (n_max > 0 && (!K || !V)) return fail(c, HKV_ERR_INVALID_ARG, f + ": K or V is NULL");
    if (n_max > 0 && (!aligned(K, 16) || !aligned(V, 16)))
        return fail(c, HKV_ERR_INVALID_ARG, f + ": K and V must be 16-byte aligned");
    const bool query = c->lay.prefill_policy == HKV_PREFILL_QUERY;
    const bool chunked = c->lay.prefill_policy == HKV_PREFILL_CHUNK;
    if (query && n_max > 0 && (!Q || !aligned(Q, 16)))
        return fail(c, HKV_ERR_INVALID_ARG, f + ": Q is NULL or not 16-byte aligned");
    if (chunked) {
        bool over = false;
        for (int b = 0; b < c->lay.B; ++b) over = over || prompt_lens[b] > c->budgets[b];
        if (over && !Q && !reuse)
            return fail(c, HKV_ERR_INVALID_ARG,
                        f + ": q_obs and reuse are both NULL while a prompt exceeds its budget");
        if ((Q && !aligned(Q, 4)) || (reuse && !aligned(reuse, 4)) || (kept && !aligned(kept, 4)))
            return fail(c, HKV_ERR_INVALID_ARG, f + ": q_obs, reuse and kept must be 4-byte aligned");
    }
    hipStream_t st = (hipStream_t)stream;
    c->plens.assign(prompt_lens, prompt_lens + c->lay.B);
    hipError_t e = hipMemcpyAsync((void*)c->dev.plen, c->plens.data(), (size_t)c->lay.B * sizeof(int32_t),
                                  hipMemcpyHostToDevice, st);
    if (e == hipSuccess) e = hipStreamSynchronize(st);   // plens is host memory of the handle
    if (e == hipSuccess)
        e = chunked ? hkv::launch_prefill_chunks(c->dev, K, V, Q, reuse, kept, chunk_list_len(c->lay), n_max, st)
                    : hkv::launch_prefill(c->dev, K, V, Q, n_max, c->lay.prefill_policy, st);
    hkv_status s = check_launch(c, e, st, fn);
    if (s != HKV_OK) return s;
    c->last_n_max = n_max;
    c->last_query_prefill = query;
    c->obs_codes = chunked && Q;
    c->prefilled = true;
    return HKV_OK;
}

extern "C" hkv_status hkv_prefill(hkv_cache* c, const void* K, const void* V, const int32_t* prompt_lens,
                                  int32_t n_max, void* stream)
{
    hkv_status s = usable(c);
    if (s != HKV_OK) return s;
    if (c->lay.prefill_policy == HKV_PREFILL_QUERY)
        return fail(c, HKV_ERR_INVALID_ARG, "hkv_prefill: this cache uses HKV_PREFILL_QUERY; call hkv_prefill_queries");
    if (c->lay.prefill_policy == HKV_PREFILL_CHUNK)
        return fail(c, HKV_ERR_INVALID_ARG, "hkv_prefill: this cache uses HKV_PREFILL_CHUNK; call hkv_prefill_chunks");
    return prefill_impl(c, K, V, nullptr, prompt_lens, n_max, stream, "hkv_prefill");
}

extern "C" hkv_status hkv_prefill_queries(hkv_cache* c, const void* K, const void* V, const float* Q,
                                          const int32_t* prompt_lens, int32_t n_max, void* stream)
{
    hkv_status s = usable(c);
    if (s != HKV_OK) return s;
    if (c->lay.prefill_policy != HKV_PREFILL_QUERY)
        return fail(c, HKV_ERR_INVALID_ARG, "hkv_prefill_queries: this cache was not created with HKV_PREFILL_QUERY");
    return prefill_impl(c, K, V, Q, prompt_lens, n_max, stream, "hkv_prefill_queries");
}

extern "C" hkv_status hkv_prefill_chunks(hkv_cache* c, const void* K, const void* V, const float* q_obs,
                                         const int32_t* reuse, int32_t* kept, const int32_t* prompt_lens,
                                         int32_t n_max, void* stream)
{
    hkv_status s = usable(c);
    if (s != HKV_OK) return s;
    if (c->lay.prefill_policy != HKV_PREFILL_CHUNK)
        return fail(c, HKV_ERR_INVALID_ARG, "hkv_prefill_chunks: this cache was not created with HKV_PREFILL_CHUNK");
    return prefill_impl(c, K, V, q_obs, prompt_lens, n_max, stream, "hkv_prefill_chunks", reuse, kept);
}

// Device address of a buffer the GPU can reach: device memory of `device` as
// is, pinned host memory through hipHostGetDevicePointer; null for anything
// else.
static void* gpu_address(void* p, int device)
{
    hipPointerAttribute_t a;
    if (hipPointerGetAttributes(&a, p) != hipSuccess) {
        (void)hipGetLastError();
        return nullptr;
    }
    if (a.type == hipMemoryTypeDevice) return a.device == device ? p : nullptr;
    if (a.type == hipMemoryTypeHost) {
        void* d = nullptr;
        if (hipHostGetDevicePointer(&d, p, 0) != hipSuccess) {
            (void)hipGetLastError();
            return nullptr;
        }
        return d;
    }
    return nullptr;
}

extern "C" hkv_status hkv_attach_tier(hkv_cache* c, void* K, void* V, int32_t* tok, void* stream)
{
    hkv_status s = usable(c);
    if (s != HKV_OK) return s;
    if (c->lay.tcap <= 0)
        return fail(c, HKV_ERR_INVALID_ARG, "hkv_attach_tier: the cache was created with tier_capacity 0");
    if (c->prefilled) return fail(c, HKV_ERR_STATE, "hkv_attach_tier: attach the tier before the prefill");
    if (!K || !V || !tok) return fail(c, HKV_ERR_INVALID_ARG, "hkv_attach_tier: NULL buffer");
    if (!aligned(K, 16) || !aligned(V, 16) || !aligned(tok, 4))
        return fail(c, HKV_ERR_INVALID_ARG, "hkv_attach_tier: K and V must be 16-byte aligned, tok 4-byte aligned");
    void* dk = gpu_address(K, c->device);
    void* dv = gpu_address(V, c->device);
    void* dt = gpu_address(tok, c->device);
    if (!dk || !dv || !dt)
        return fail(c, HKV_ERR_INVALID_ARG,
                    "hkv_attach_tier: tier buffers must be pinned host memory (hipHostMalloc) or memory of the "
                    "cache's device");
    hipStream_t st = (hipStream_t)stream;
    hipError_t e = hipMemsetAsync(c->dev.tcount, 0, (size_t)c->lay.B * c->lay.Hkv * 4, st);
    s = check_launch(c, e, st, "hkv_attach_tier");
    if (s != HKV_OK) return s;
    c->dev.tK = dk;
    c->dev.tV = dv;
    c->dev.ttok = (int*)dt;
    return HKV_OK;
}

extern "C" hkv_status hkv_tier_counts(const hkv_cache* cc, int32_t* counts, void* stream)
{
    hkv_cache* c = const_cast<hkv_cache*>(cc);
    hkv_status s = usable(c);
    if (s != HKV_OK) return s;
    if (!c->dev.tK) return fail(c, HKV_ERR_STATE, "hkv_tier_counts: no tier attached");
    if (!counts) return fail(c, HKV_ERR_INVALID_ARG, "hkv_tier_counts: counts is NULL");
    hipStream_t st = (hipStream_t)stream;
    hipError_t e = hipMemcpyAsync(counts, c->dev.tcount, (size_t)c->lay.B * c->lay.Hkv * 4, hipMemcpyDefault, st);
    return check_launch(c, e, st, "hkv_tier_counts");
}

extern "C" hkv_status hkv_attend_tiered(hkv_cache* c, const float* q, float* out, void* stream)
{
    hkv_status s = usable(c);
    if (s != HKV_OK) return s;
    if (!c->dev.tK) return fail(c, HKV_ERR_STATE, "hkv_attend_tiered: no tier attached");
    if (!c->prefilled) return fail(c, HKV_ERR_STATE, "hkv_attend_tiered: call hkv_prefill* or hkv_set_state first");
    if (!q || !out) return fail(c, HKV_ERR_INVALID_ARG, "hkv_attend_tiered: NULL buffer");
    if (!aligned(q, 16) || !aligned(out, 16))
        return fail(c, HKV_ERR_INVALID_ARG, "hkv_attend_tiered: q and out must be 16-byte aligned");
    hipStream_t st = (hipStream_t)stream;
    hipError_t e = c->debug_nan ? hkv::launch_poison_partials(c->dev, st) : hipSuccess;
    if (e == hipSuccess) e = hkv::launch_attend_tiered(c->dev, q, out, st);
    return check_launch(c, e, st, "hkv_attend_tiered");
}

extern "C" hkv_status hkv_decode_step(hkv_cache* c, const float* q, const void* k, const void* v,
                                      float* out, int32_t* evicted_slot, void* stream)
{
    hkv_status s = usable(c);
    if (s != HKV_OK) return s;
    if (!c->prefilled) return fail(c, HKV_ERR_STATE, "hkv_decode_step: call hkv_prefill or hkv_set_state first");
    if (!q || !k || !v || !out || !evicted_slot)
        return fail(c, HKV_ERR_INVALID_ARG, "hkv_decode_step: NULL buffer");
    if (!aligned(q, 16) || !aligned(k, 16) || !aligned(v, 16))
        return fail(c, HKV_ERR_INVALID_ARG, "hkv_decode_step: q, k, v must be 16-byte aligned");
    hipStream_t st = (hipStream_t)stream;
    hipError_t e = c->debug_nan ? hkv::launch_poison_partials(c->dev, st) : hipSuccess;
    if (e == hipSuccess)
        e = c->lay.schedule == HKV_DECODE_FUSED ? hkv::launch_decode_fused(c->dev, q, k, v, out, evicted_slot, st)
                                                : hkv::launch_decode_split(c->dev, q, k, v, out, evicted_slot, st);
    s = check_launch(c, e, st, "hkv_decode_step");
    if (s == HKV_OK) {
        c->stepped = true;
        c->obs_codes = false;
    }
    return s;
}

extern "C" hkv_status hkv_decode_step_static(hkv_cache* c, const float* q, const void* k, const void* v,
                                             float* out, int32_t* evicted_slot, void* stream)
{
    hkv_status s = usable(c);
    if (s != HKV_OK) return s;
    if (!c->prefilled)
        return fail(c, HKV_ERR_STATE, "hkv_decode_step_static: call hkv_prefill or hkv_set_state first");
    if (!q || !k || !v || !out || !evicted_slot)
        return fail(c, HKV_ERR_INVALID_ARG, "hkv_decode_step_static: NULL buffer");
    if (!aligned(q, 16) || !aligned(k, 16) || !aligned(v, 16))
        return fail(c, HKV_ERR_INVALID_ARG, "hkv_decode_step_static: q, k, v must be 16-byte aligned");
    const size_t need = carve_step_scratch(c->lay, nullptr, nullptr);
    if (need > kStaticScratchBytes) {
        char msg[200];
        snprintf(msg, sizeof(msg),
                 "hkv_decode_step_static: this cache's step needs %zu bytes of scratch, more than the %zu of the "
                 "static scratch (fewer splits, i.e. a larger chunk, or hkv_decode_step)", need, kStaticScratchBytes);
        return fail(c, HKV_ERR_UNSUPPORTED, msg);
    }
    char* base = (char*)static_scratch(c->device);
    if (!base) return fail(c, HKV_ERR_STATE, "hkv_decode_step_static: no static scratch on this device");
    hkv::DevCache d = c->dev;
    carve_step_scratch(c->lay, base, &d);
    hipStream_t st = (hipStream_t)stream;
    // the array keeps the last call's contents: the eviction keys and ticket
    // counters must start at zero (a kernel, not a memset, so the step can be
    // captured in a graph)
    hipError_t e = hkv::launch_clear_step_scratch(d, st);
    if (e == hipSuccess && c->debug_nan) e = hkv::launch_poison_partials(d, st);
    if (e == hipSuccess)
        e = c->lay.schedule == HKV_DECODE_FUSED ? hkv::launch_decode_fused(d, q, k, v, out, evicted_slot, st)
                                                : hkv::launch_decode_split(d, q, k, v, out, evicted_slot, st);
    s = check_launch(c, e, st, "hkv_decode_step_static");
    if (s == HKV_OK) {
        c->stepped = true;
        c->obs_codes = false;
    }
    return s;
}

extern "C" hkv_status hkv_get_state(const hkv_cache* cc, void* K, void* V, uint32_t* codes,
                                    int32_t* slot_token, int32_t* head_state, void* stream)
{
    hkv_cache* c = const_cast<hkv_cache*>(cc);
    hkv_status s = usable(c);
    if (s != HKV_OK) return s;
    const hkv::Layout& L = c->lay;
    hipStream_t st = (hipStream_t)stream;
    const size_t heads = (size_t)L.B * L.Hkv;
    const size_t kv = heads * L.Smax * L.d * L.es;
    hipError_t e = hipSuccess;
    if (K) e = hipMemcpyAsync(K, c->dev.K, kv, hipMemcpyDeviceToDevice, st);
    if (e == hipSuccess && V) e = hipMemcpyAsync(V, c->dev.V, L.v_bytes, hipMemcpyDeviceToDevice, st);
    if (e == hipSuccess && V && L.value_bits != 0)
        e = hipMemcpyAsync((char*)V + L.v_bytes, c->dev.vs, heads * L.Smax * 4, hipMemcpyDeviceToDevice, st);
    if (e == hipSuccess && codes) e = hkv::launch_export_codes(c->dev, codes, st);
    if (e == hipSuccess && slot_token)
        e = hipMemcpyAsync(slot_token, c->dev.tok, heads * L.Smax * 4, hipMemcpyDeviceToDevice, st);
    if (e == hipSuccess && head_state)
        e = hipMemcpyAsync(head_state, c->dev.state, heads * 8, hipMemcpyDeviceToDevice, st);
    return check_launch(c, e, st, "hkv_get_state");
}

extern "C" hkv_status hkv_set_state(hkv_cache* c, const void* K, const void* V, const uint32_t* codes,
                                    const int32_t* slot_token, const int32_t* head_state, void* stream)
{
    hkv_status s = usable(c);
    if (s != HKV_OK) return s;
    if (!K || !V || !codes || !slot_token || !head_state)
        return fail(c, HKV_ERR_INVALID_ARG, "hkv_set_state: all five buffers are required");
    const hkv::Layout& L = c->lay;
    hipStream_t st = (hipStream_t)stream;
    const size_t heads = (size_t)L.B * L.Hkv;
    const size_t kv = heads * L.Smax * L.d * L.es;
    // The occupancy and position of every head decide which slots the kernels
    // read and write, so they are checked on the host before anything is
    // enqueued: 0 <= occupancy <= budget and occupancy <= position.
    std::vector<int32_t> hs(heads * 2);
    hipError_t e = hipMemcpyAsync(hs.data(), head_state, heads * 8, hipMemcpyDeviceToHost, st);
    if (e == hipSuccess) e = hipStreamSynchronize(st);
    if (e != hipSuccess) return check_launch(c, e, st, "hkv_set_state");
    for (size_t i = 0; i < heads; ++i) {
        const int32_t n = hs[2 * i], t = hs[2 * i + 1], S = c->budgets[i / L.Hkv];
        if (n < 0 || n > S || t < n) {
            char msg[160];
            snprintf(msg, sizeof(msg), "hkv_set_state: head_state of sequence %zu, KV head %zu is (%d, %d); needs "
                     "0 <= occupancy <= budget %d and occupancy <= position", i / L.Hkv, i % L.Hkv, n, t, S);
            return fail(c, HKV_ERR_INVALID_ARG, msg);
        }
    }
    e = hipMemcpyAsync(c->dev.K, K, kv, hipMemcpyDeviceToDevice, st);
    if (e == hipSuccess) e = hipMemcpyAsync(c->dev.V, V, L.v_bytes, hipMemcpyDeviceToDevice, st);
    if (e == hipSuccess && L.value_bits != 0)
        e = hipMemcpyAsync(c->dev.vs, (const char*)V + L.v_bytes, heads * L.Smax * 4, hipMemcpyDeviceToDevice, st);
    if (e == hipSuccess) e = hkv::launch_import_codes(c->dev, codes, st);
    if (e == hipSuccess) e = hipMemcpyAsync(c->dev.tok, slot_token, heads * L.Smax * 4, hipMemcpyDeviceToDevice, st);
    if (e == hipSuccess) e = hipMemcpyAsync(c->dev.state, head_state, heads * 8, hipMemcpyDeviceToDevice, st);
    if (e == hipSuccess) e = hkv::launch_clear_step_scratch(c->dev, st);
    s = check_launch(c, e, st, "hkv_set_state");
    if (s == HKV_OK) {
        c->prefilled = true;
        c->last_query_prefill = false;
        c->obs_codes = false;
    }
    return s;
}

extern "C" hkv_status hkv_debug_last_codes(const hkv_cache* cc, uint32_t* qcodes, uint32_t* kcodes, void* stream)
{
    hkv_cache* c = const_cast<hkv_cache*>(cc);
    hkv_status s = usable(c);
    if (s != HKV_OK) return s;
    if (!c->stepped && !c->obs_codes)
        return fail(c, HKV_ERR_STATE, "hkv_debug_last_codes: no decode step (or observed chunk prefill) yet");
    const hkv::Layout& L = c->lay;
    hipStream_t st = (hipStream_t)stream;
    hipError_t e = hipSuccess;
    if (qcodes) e = hipMemcpyAsync(qcodes, c->dev.dbg_q, (size_t)L.B * L.Hq * L.W * 4, hipMemcpyDeviceToDevice, st);
    if (e == hipSuccess && kcodes)
        e = hipMemcpyAsync(kcodes, c->dev.dbg_k, (size_t)L.B * L.Hkv * L.W * 4, hipMemcpyDeviceToDevice, st);
    return check_launch(c, e, st, "hkv_debug_last_codes");
}

extern "C" hkv_status hkv_debug_prefill_codes(const hkv_cache* cc, uint32_t* codes, void* stream)
{
    hkv_cache* c = const_cast<hkv_cache*>(cc);
    hkv_status s = usable(c);
    if (s != HKV_OK) return s;
    if (!c->prefilled) return fail(c, HKV_ERR_STATE, "hkv_debug_prefill_codes: no prefill yet");
    if (!codes) return fail(c, HKV_ERR_INVALID_ARG, "hkv_debug_prefill_codes: codes is NULL");
    hipStream_t st = (hipStream_t)stream;
    return check_launch(c, hkv::launch_export_pcodes(c->dev, codes, c->last_n_max, false, st), st,
                        "hkv_debug_prefill_codes");
}

extern "C" hkv_status hkv_debug_prefill_query_codes(const hkv_cache* cc, uint32_t* codes, void* stream)
{
    hkv_cache* c = const_cast<hkv_cache*>(cc);
    hkv_status s = usable(c);
    if (s != HKV_OK) return s;
    if (!c->prefilled || !c->last_query_prefill)
        return fail(c, HKV_ERR_STATE, "hkv_debug_prefill_query_codes: no QUERY prefill yet");
    if (!codes) return fail(c, HKV_ERR_INVALID_ARG, "hkv_debug_prefill_query_codes: codes is NULL");
    hipStream_t st = (hipStream_t)stream;
    return check_launch(c, hkv::launch_export_pcodes(c->dev, codes, c->last_n_max, true, st), st,
                        "hkv_debug_prefill_query_codes");
}

extern "C" hkv_status hkv_debug_scores(const hkv_cache* cc, const uint32_t* qcodes, int32_t* scores, void* stream)
{
    hkv_cache* c = const_cast<hkv_cache*>(cc);
    hkv_status s = usable(c);
    if (s != HKV_OK) return s;
    if (!qcodes || !scores) return fail(c, HKV_ERR_INVALID_ARG, "hkv_debug_scores: NULL buffer");
    hipStream_t st = (hipStream_t)stream;
    return check_launch(c, hkv::launch_scores(c->dev, qcodes, scores, st), st, "hkv_debug_scores");
}

extern "C" hkv_status hkv_encode(const hkv_cache* cc, const void* X, int32_t x_dtype, int32_t n,
                                 uint32_t* codes, void* stream)
{
    hkv_cache* c = const_cast<hkv_cache*>(cc);
    hkv_status s = usable(c);
    if (s != HKV_OK) return s;
    if (n < 0) return fail(c, HKV_ERR_INVALID_ARG, "hkv_encode: n < 0");
    if (x_dtype != HKV_F32 && x_dtype != HKV_BF16) return fail(c, HKV_ERR_UNSUPPORTED, "hkv_encode: x_dtype");
    if (n > 0 && (!X || !codes)) return fail(c, HKV_ERR_INVALID_ARG, "hkv_encode: NULL buffer");
    hipStream_t st = (hipStream_t)stream;
    return check_launch(c, hkv::launch_encode_rows(c->dev, X, x_dtype == HKV_BF16, n, codes, st), st,
                        "hkv_encode");
}
