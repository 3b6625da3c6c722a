// fa_api.cpp - the C ABI of libfa_mi355x: argument checks, variant selection
// and launch on the caller's stream.  See include/fa_mi355x.h for the
// contract of every entry point.
//
// The checks follow mlx-native flash_attn_train.rs (validate_params: every
// size positive, H_q divisible by H_kv; dispatch_inner: head_dim and dtype
// checks before any launch) and add this library's own pointer, alignment
// and stride rules.  Everything is checked before anything is launched.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <cmath>
#include <cstdarg>
#include <cstdint>
#include <cstdio>
#include <cstring>

#include <map>
#include <mutex>
#include <utility>
#include <vector>

#include "fa_common.h"
#include "fa_mi355x.h"

namespace fa {

namespace {

// The per-head-dim tables of one kind, concatenated once.
typedef const Variant* (*TableFn)(int*);
const Variant* concat_tables(const TableFn* fns, int nfns, std::vector<Variant>& all, std::once_flag& once, int* n)
{
    std::call_once(once, [&]() {
        for (int i = 0; i < nfns; ++i) {
            int k = 0;
            const Variant* t = fns[i](&k);
            all.insert(all.end(), t, t + k);
        }
    });
    *n = (int)all.size();
    return all.data();
}

}  // namespace

#define FA_TABLE_OF(KIND)                                               \
    const Variant* variants_##KIND(int* n)                              \
    {                                                                   \
        static const TableFn fns[] = {                                  \
            variants_##KIND##_d16, variants_##KIND##_d32,  variants_##KIND##_d48, variants_##KIND##_d64, \
            variants_##KIND##_d80, variants_##KIND##_d96, variants_##KIND##_d128, variants_##KIND##_d256}; \
        static std::vector<Variant> all;                                \
        static std::once_flag once;                                     \
        return concat_tables(fns, 8, all, once, n);                     \
    }
FA_TABLE_OF(bf16)
FA_TABLE_OF(f32)
FA_TABLE_OF(bf16_dropout)
FA_TABLE_OF(f32_dropout)
#undef FA_TABLE_OF

const BwdVariant* bwd_variants_bf16(int* n)
{
    static std::vector<BwdVariant> all;
    static std::once_flag once;
    std::call_once(once, []() {
        const BwdVariant* (*fns[])(int*) = {bwd_variants_bf16_d64, bwd_variants_bf16_d128};
        for (auto fn : fns) {
            int k = 0;
            const BwdVariant* t = fn(&k);
            all.insert(all.end(), t, t + k);
        }
    });
    *n = (int)all.size();
    return all.data();
}

// Partials of split launches come from a stream-ordered memory pool that the
// library creates for itself, one per device.  The process-wide default pool
// and its attributes are left alone.  This pool keeps up to kPoolKeepBytes of
// freed memory for reuse instead of returning it at every synchronisation.
hipError_t library_pool(hipMemPool_t* out)
{
    constexpr uint64_t kPoolKeepBytes = 256ull << 20;
    constexpr int kMaxDevices = 64;
    static std::once_flag once[kMaxDevices];
    static hipMemPool_t pools[kMaxDevices];
    static hipError_t status[kMaxDevices];
    int dev = 0;
    const hipError_t err = hipGetDevice(&dev);
    if (err != hipSuccess) return err;
    if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
    std::call_once(once[dev], [dev]() {
        hipMemPoolProps props;
        std::memset(&props, 0, sizeof(props));
        props.allocType = hipMemAllocationTypePinned;
        props.handleTypes = hipMemHandleTypeNone;
        props.location.type = hipMemLocationTypeDevice;
        props.location.id = dev;
        status[dev] = hipMemPoolCreate(&pools[dev], &props);
        if (status[dev] == hipSuccess) {
            uint64_t keep = kPoolKeepBytes;
            status[dev] = hipMemPoolSetAttribute(pools[dev], hipMemPoolAttrReleaseThreshold, &keep);
        }
    });
    *out = pools[dev];
    return status[dev];
}

// Partials of a split forward launch: a workspace the library keeps per
// (device, stream), taken from its pool and grown when a launch needs more
// than it holds.  An allocation and a free from the pool per call cost the
// host ~30 us, as much as a whole decode-sized launch on the GPU.  Every use
// waits on the stream for an event recorded after the previous use of the
// same workspace, so reuse stays ordered even when a stream handle is
// destroyed and handed out again; the mutex is held from that wait to the
// event record, so uses from several host threads are ordered too.  The
// event skips the system-scope fence (it only orders work on this device):
// a default event record cost ~2.8 us of GPU time per call, this one ~0.9.
// A workspace is held until the process ends; a device keeps at most
// kMaxStreams of them, and calls on further streams allocate from the pool
// per call, as before.
struct StreamWorkspace {
    void* ptr = nullptr;
    size_t bytes = 0;
    hipEvent_t done = nullptr;
};

std::mutex& workspace_mutex()
{
    static std::mutex mu;
    return mu;
}

// Launch `var` with its partials in the workspace of (current device, st);
// the caller holds workspace_mutex().
hipError_t launch_with_workspace(const Variant* var, FwdParams p, hipStream_t st, size_t need)
{
    static std::map<std::pair<int, hipStream_t>, StreamWorkspace> spaces;
    static std::map<int, int> per_device;  // workspaces held per device
    constexpr size_t kGrain = 1u << 20;    // grown in whole MiB
    constexpr int kMaxStreams = 8;
    int dev = 0;
    hipError_t err = hipGetDevice(&dev);
    if (err != hipSuccess) return err;
    const auto key = std::make_pair(dev, st);
    if (spaces.find(key) == spaces.end()) {
        if (per_device[dev] >= kMaxStreams) return var->launch(p, st, nullptr);  // the pool, per call
        ++per_device[dev];
    }
    StreamWorkspace& w = spaces[key];
    if (w.done == nullptr) {
        err = hipEventCreateWithFlags(&w.done, hipEventDisableTiming | hipEventDisableSystemFence);
        if (err != hipSuccess) {
            w.done = nullptr;
            return err;
        }
    } else {
        err = hipStreamWaitEvent(st, w.done, 0);
        if (err != hipSuccess) return err;
    }
    if (w.bytes < need) {
        hipMemPool_t pool;
        err = library_pool(&pool);
        if (err != hipSuccess) return err;
        if (w.ptr != nullptr) {
            err = hipFreeAsync(w.ptr, st);
            w.ptr = nullptr;
            w.bytes = 0;
            if (err != hipSuccess) return err;
        }
        const size_t bytes = (need + kGrain - 1) / kGrain * kGrain;
        err = hipMallocFromPoolAsync(&w.ptr, bytes, pool, st);
        if (err != hipSuccess) {
            w.ptr = nullptr;
            return err;
        }
        w.bytes = bytes;
    }
    p.ws = (float*)w.ptr;
    p.ws_bytes = w.bytes;
    err = var->launch(p, st, nullptr);
    const hipError_t rerr = hipEventRecord(w.done, st);
    return err != hipSuccess ? err : rerr;
}

// Scratch of fa_fwd_strided_noalloc: the partials of a split key range.
// The split plan fills the GPU once, so n_split * (rows of the launch) is at
// most 256 CUs x 8 resident waves x 32 rows = 65536, and the partials
// (n_split * rows * (D + 1) fp32) at most 65536 * 257 * 4 bytes at D = 256
// and 65536 * 129 * 4 bytes at D = 128: under kScratchBytes for every shape
// (the size is still checked before each launch).  One copy per GPU, in the
// library's device image, held until the process ends.  Host code never
// passes `scratch` itself to a kernel (in host code the name is only a
// stand-in): it uses the device address hipGetSymbolAddress gives for it.
constexpr size_t kScratchBytes = 36ull << 20;
static_assert(kScratchBytes == FA_NOALLOC_SCRATCH_BYTES, "the header states the scratch size");
static __device__ __align__(256) float scratch[kScratchBytes / sizeof(float)];

// The device address of `scratch` on the current device, looked up once per
// device with that device current.
hipError_t scratch_address(float** out)
{
    constexpr int kMaxDevices = 64;
    static std::once_flag once[kMaxDevices];
    static float* ptrs[kMaxDevices];
    static hipError_t status[kMaxDevices];
    int dev = 0;
    const hipError_t err = hipGetDevice(&dev);
    if (err != hipSuccess) return err;
    if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
    std::call_once(once[dev], [dev]() {
        void* ptr = nullptr;
        status[dev] = hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch));
        ptrs[dev] = (float*)ptr;
    });
    *out = ptrs[dev];
    return status[dev];
}

}  // namespace fa

namespace {

thread_local char g_last_error[512] = "";

fa_status fail(fa_status st, const char* fmt, ...)
{
    va_list ap;
    va_start(ap, fmt);
    vsnprintf(g_last_error, sizeof(g_last_error), fmt, ap);
    va_end(ap);
    return st;
}

// Dropout of a fa_fwd_dropout call.
struct DropArgs {
    float p;
    uint64_t seed, offset;
};

const fa::Variant* find_variant(int dtype, int D, int mask, int causal, bool dropout = false)
{
    int n = 0;
    const fa::Variant* tab = dropout ? (dtype == FA_DTYPE_BF16 ? fa::variants_bf16_dropout(&n) : fa::variants_f32_dropout(&n))
                             : dtype == FA_DTYPE_BF16 ? fa::variants_bf16(&n) : fa::variants_f32(&n);
    for (int i = 0; i < n; ++i)
        if (tab[i].D == D && tab[i].mask == mask && tab[i].causal == (causal ? 1 : 0)) return &tab[i];
    return nullptr;
}

bool aligned(const void* ptr, uintptr_t a) { return ((uintptr_t)ptr % a) == 0; }

bool all_zero(const int64_t s[3]) { return s[0] == 0 && s[1] == 0 && s[2] == 0; }

// Contiguous default {batch, head, seq} strides of a [B, H, L, inner] tensor.
void default_strides(int64_t out[3], int64_t H, int64_t Lx, int64_t inner)
{
    out[2] = inner;
    out[1] = Lx * inner;
    out[0] = H * Lx * inner;
}

}  // namespace

extern "C" {

const char* fa_status_string(fa_status s)
{
    switch (s) {
    case FA_OK: return "FA_OK";
    case FA_ERR_INVALID_ARGUMENT: return "FA_ERR_INVALID_ARGUMENT";
    case FA_ERR_UNSUPPORTED: return "FA_ERR_UNSUPPORTED";
    case FA_ERR_HIP: return "FA_ERR_HIP";
    }
    return "FA_ERR_UNKNOWN";
}

const char* fa_last_error(void) { return g_last_error; }

int fa_abi_version(void) { return FA_ABI_VERSION; }

// Every compiled variant: the bf16 and fp32 tables, then their dropout tables.
static const fa::Variant* variant_table(int which, int* n)
{
    switch (which) {
    case 0: return fa::variants_bf16(n);
    case 1: return fa::variants_f32(n);
    case 2: return fa::variants_bf16_dropout(n);
    case 3: return fa::variants_f32_dropout(n);
    }
    *n = 0;
    return nullptr;
}

int fa_variant_count(void)
{
    int total = 0;
    for (int w = 0; w < 4; ++w) {
        int n = 0;
        variant_table(w, &n);
        total += n;
    }
    int nb = 0;
    fa::bwd_variants_bf16(&nb);
    return total + nb;
}

const char* fa_variant_name(int i)
{
    if (i < 0) return nullptr;
    for (int w = 0; w < 4; ++w) {
        int n = 0;
        const fa::Variant* t = variant_table(w, &n);
        if (i < n) return t[i].name;
        i -= n;
    }
    int nb = 0;
    const fa::BwdVariant* tb = fa::bwd_variants_bf16(&nb);
    return i < nb ? tb[i].name : nullptr;
}

static const fa::BwdVariant* find_bwd_variant(int dtype, int D, int mask, int causal)
{
    if (dtype != FA_DTYPE_BF16) return nullptr;
    int n = 0;
    const fa::BwdVariant* t = fa::bwd_variants_bf16(&n);
    for (int i = 0; i < n; ++i)
        if (t[i].D == D && t[i].mask == mask && t[i].causal == (causal ? 1 : 0)) return &t[i];
    return nullptr;
}

int fa_bwd_supported(fa_dtype dtype, int D, fa_mask_kind mask_kind, int causal)
{
    return find_bwd_variant(dtype, D, mask_kind, causal) != nullptr;
}

int fa_supported(fa_dtype dtype, int D, fa_mask_kind mask_kind, int causal)
{
    if (dtype != FA_DTYPE_F32 && dtype != FA_DTYPE_BF16) return 0;
    if (mask_kind < FA_MASK_NONE || mask_kind > FA_MASK_BOOL) return 0;
    return find_variant(dtype, D, mask_kind, causal) != nullptr;
}

}  // extern "C"

namespace {

fa_status fwd_impl(const void* Q, const void* K, const void* V, const void* mask,
                   void* O, float* L,
                   int B, int H_q, int H_kv, int qL, int kL, int D,
                   float scale, int causal,
                   fa_dtype dtype, fa_mask_kind mask_kind,
                   const fa_strides* strides, void* hip_stream, const DropArgs* drop, int window = 0,
                   bool noalloc = false)
{
    g_last_error[0] = '\0';
    const fa_status E = FA_ERR_INVALID_ARGUMENT;
    if (B <= 0) return fail(E, "fa_fwd: B must be > 0, got %d", B);
    if (H_q <= 0) return fail(E, "fa_fwd: H_q must be > 0, got %d", H_q);
    if (H_kv <= 0) return fail(E, "fa_fwd: H_kv must be > 0, got %d", H_kv);
    if (H_q % H_kv != 0) return fail(E, "fa_fwd: H_q (%d) must be divisible by H_kv (%d)", H_q, H_kv);
    if (qL <= 0) return fail(E, "fa_fwd: qL must be > 0, got %d", qL);
    if (kL <= 0) return fail(E, "fa_fwd: kL must be > 0, got %d", kL);
    if (D != 16 && D != 32 && D != 48 && D != 64 && D != 80 && D != 96 && D != 128 && D != 256)
        return fail(E, "fa_fwd: D must be 16, 32, 48, 64, 80, 96, 128 or 256, got %d", D);
    if (dtype != FA_DTYPE_F32 && dtype != FA_DTYPE_BF16) return fail(E, "fa_fwd: unknown dtype %d", (int)dtype);
    if (mask_kind != FA_MASK_NONE && mask_kind != FA_MASK_ADDITIVE && mask_kind != FA_MASK_BOOL)
        return fail(E, "fa_fwd: unknown mask kind %d", (int)mask_kind);
    if ((mask_kind == FA_MASK_NONE) != (mask == nullptr))
        return fail(E, "fa_fwd: mask must be NULL exactly when mask_kind is FA_MASK_NONE");
    if (!Q || !K || !V || !O || !L) return fail(E, "fa_fwd: Q, K, V, O and L must be non-NULL");
    if (!std::isfinite(scale)) return fail(E, "fa_fwd: scale must be finite");
    if (drop && !(drop->p >= 0.f && drop->p <= 1.f))
        return fail(E, "fa_fwd_dropout: the dropout rate must lie in [0, 1], got %g", (double)drop->p);
    if (window < 0) return fail(E, "fa_fwd_window: the window must be >= 1 key, got %d", window);
    if (window > 0 && !causal) return fail(E, "fa_fwd_window: a sliding window needs causal = 1");
    if (!aligned(Q, 16) || !aligned(K, 16) || !aligned(V, 16) || !aligned(O, 16) || !aligned(L, 4))
        return fail(E, "fa_fwd: Q, K, V and O must be 16-byte aligned and L 4-byte aligned");
    if ((int64_t)B * H_q * qL * D > INT64_MAX / 8 || (int64_t)B * H_q * qL * kL > INT64_MAX / 8)
        return fail(E, "fa_fwd: tensor too large");

    const int esz = dtype == FA_DTYPE_BF16 ? 2 : 4;
    const int vec_elems = 16 / esz;
    fa::FwdParams p;
    std::memset(&p, 0, sizeof(p));
    p.n_split = 1;  // the kernels divide the grid by it: never 0
    p.window = window;
    if (drop) {
        p.drop_p = drop->p;
        p.drop_scale = drop->p < 1.f ? 1.f / (1.f - drop->p) : 0.f;
        // p 2^24 is exact in fp32 (a power-of-two scaling), so its ceiling is
        // the smallest kept floor(w / 2^8); p = 1 wraps to 0 and is dropped
        // through drop_scale = 0 instead
        p.drop_thresh = (uint32_t)std::ceil((double)drop->p * 16777216.0) << 8;
        p.seed_lo = (uint32_t)drop->seed;
        p.seed_hi = (uint32_t)(drop->seed >> 32);
        p.off_lo = (uint32_t)drop->offset;
        p.off_hi = (uint32_t)(drop->offset >> 32);
    }
    fa_strides s;
    if (strides) s = *strides;
    else std::memset(&s, 0, sizeof(s));
    if (all_zero(s.q)) default_strides(s.q, H_q, qL, D);
    if (all_zero(s.k)) default_strides(s.k, H_kv, kL, D);
    if (all_zero(s.v)) default_strides(s.v, H_kv, kL, D);
    if (all_zero(s.o)) default_strides(s.o, H_q, qL, D);
    if (all_zero(s.mask)) default_strides(s.mask, H_q, qL, kL);
    const struct { const int64_t* st; const char* name; } t4[] = {{s.q, "Q"}, {s.k, "K"}, {s.v, "V"}, {s.o, "O"}};
    for (const auto& t : t4)
        for (int a = 0; a < 3; ++a)
            if (t.st[a] < 0 || t.st[a] % vec_elems != 0)
                return fail(E, "fa_fwd: %s stride %d (%lld) must be a non-negative multiple of %d elements",
                            t.name, a, (long long)t.st[a], vec_elems);
    for (int a = 0; a < 3; ++a)
        if (s.mask[a] < 0) return fail(E, "fa_fwd: mask strides must be non-negative");

    const fa::Variant* var = find_variant(dtype, D, mask_kind, causal, drop != nullptr);
    if (!var)
        return fail(FA_ERR_UNSUPPORTED, "fa_fwd: no kernel built for dtype %d, D %d, mask %d, causal %d",
                    (int)dtype, D, (int)mask_kind, causal);

    p.q = Q;
    p.k = K;
    p.v = V;
    p.mask = mask;
    p.o = O;
    p.lse = L;
    for (int a = 0; a < 3; ++a) {
        p.q_s[a] = s.q[a];
        p.k_s[a] = s.k[a];
        p.v_s[a] = s.v[a];
        p.o_s[a] = s.o[a];
        p.m_s[a] = s.mask[a];
    }
    p.B = B;
    p.Hq = H_q;
    p.Hkv = H_kv;
    p.qL = qL;
    p.kL = kL;
    p.group = H_q / H_kv;
    p.n_qtiles = (qL + var->block_m - 1) / var->block_m;
    p.neg_q = scale < 0.f ? 1 : 0;
    p.scale_log2 = std::fabs(scale) * 1.4426950408889634f;
    if (mask_kind != FA_MASK_NONE) {
        // 4 consecutive mask entries load as one vector when every row start is
        // aligned to 4 elements' worth of bytes.
        const int mesz = mask_kind == FA_MASK_BOOL ? 1 : esz;
        const uintptr_t need = (uintptr_t)4 * mesz;
        p.mask_vec = aligned(mask, need) && s.mask[0] % 4 == 0 && s.mask[1] % 4 == 0 && s.mask[2] % 4 == 0;
    }
    if ((int64_t)p.n_qtiles * H_q * B > 0x7fffffffLL) return fail(E, "fa_fwd: grid too large");

    if (noalloc) {
        // the partials of a split launch go to the static scratch, never to
        // allocated memory; a launch that would need more is refused
        size_t need = 0;
        hipError_t perr = var->launch(p, (hipStream_t)hip_stream, &need);
        if (perr != hipSuccess) return fail(FA_ERR_HIP, "fa_fwd_strided_noalloc: planning of %s failed: %s", var->name,
                                            hipGetErrorString(perr));
        if (need > fa::kScratchBytes)
            return fail(E, "fa_fwd_strided_noalloc: this launch needs %zu bytes of scratch, more than the %zu-byte "
                        "maximum", need, fa::kScratchBytes);
        if (need > 0) {
            perr = fa::scratch_address(&p.ws);
            if (perr != hipSuccess)
                return fail(FA_ERR_HIP, "fa_fwd_strided_noalloc: no scratch on this device: %s", hipGetErrorString(perr));
            p.ws_bytes = fa::kScratchBytes;
        }
    }
    else {
        // a split launch takes its partials from the stream's workspace
        size_t need = 0;
        hipError_t perr = var->launch(p, (hipStream_t)hip_stream, &need);
        if (perr != hipSuccess)
            return fail(FA_ERR_HIP, "fa_fwd: planning of %s failed: %s", var->name, hipGetErrorString(perr));
        if (need > 0) {
            std::lock_guard<std::mutex> guard(fa::workspace_mutex());
            perr = fa::launch_with_workspace(var, p, (hipStream_t)hip_stream, need);
            if (perr != hipSuccess)
                return fail(FA_ERR_HIP, "fa_fwd: launch of %s failed: %s", var->name, hipGetErrorString(perr));
            return FA_OK;
        }
    }
    const hipError_t err = var->launch(p, (hipStream_t)hip_stream, nullptr);
    if (err != hipSuccess) return fail(FA_ERR_HIP, "fa_fwd: launch of %s failed: %s", var->name, hipGetErrorString(err));
    return FA_OK;
}

}  // namespace

extern "C" {

fa_status fa_fwd_strided(const void* Q, const void* K, const void* V, const void* mask,
                         void* O, float* L,
                         int B, int H_q, int H_kv, int qL, int kL, int D,
                         float scale, int causal,
                         fa_dtype dtype, fa_mask_kind mask_kind,
                         const fa_strides* strides, void* hip_stream)
{
    return fwd_impl(Q, K, V, mask, O, L, B, H_q, H_kv, qL, kL, D, scale, causal, dtype, mask_kind, strides,
                    hip_stream, nullptr);
}

fa_status fa_fwd_strided_noalloc(const void* Q, const void* K, const void* V, const void* mask,
                                 void* O, float* L,
                                 int B, int H_q, int H_kv, int qL, int kL, int D,
                                 float scale, int causal,
                                 fa_dtype dtype, fa_mask_kind mask_kind,
                                 const fa_strides* strides, void* hip_stream)
{
    return fwd_impl(Q, K, V, mask, O, L, B, H_q, H_kv, qL, kL, D, scale, causal, dtype, mask_kind, strides,
                    hip_stream, nullptr, 0, true);
}

fa_status fa_fwd_dropout(const void* Q, const void* K, const void* V, const void* mask,
                         void* O, float* L,
                         int B, int H_q, int H_kv, int qL, int kL, int D,
                         float scale, int causal,
                         fa_dtype dtype, fa_mask_kind mask_kind,
                         float p_drop, uint64_t seed, uint64_t offset,
                         const fa_strides* strides, void* hip_stream)
{
    const DropArgs drop{p_drop, seed, offset};
    return fwd_impl(Q, K, V, mask, O, L, B, H_q, H_kv, qL, kL, D, scale, causal, dtype, mask_kind, strides,
                    hip_stream, &drop);
}

fa_status fa_fwd_window(const void* Q, const void* K, const void* V, const void* mask,
                        void* O, float* L,
                        int B, int H_q, int H_kv, int qL, int kL, int D,
                        float scale, int causal,
                        fa_dtype dtype, fa_mask_kind mask_kind,
                        int window, const fa_strides* strides, void* hip_stream)
{
    if (window < 1) {
        g_last_error[0] = '\0';
        return fail(FA_ERR_INVALID_ARGUMENT, "fa_fwd_window: the window must be >= 1 key, got %d", window);
    }
    return fwd_impl(Q, K, V, mask, O, L, B, H_q, H_kv, qL, kL, D, scale, causal, dtype, mask_kind, strides,
                    hip_stream, nullptr, window);
}

fa_status fa_bwd(const void* Q, const void* K, const void* V, const void* O, const void* dO, const float* L,
                 const void* mask, float* Delta, void* dQ, void* dK, void* dV,
                 int B, int H_q, int H_kv, int qL, int kL, int D,
                 float scale, int causal,
                 fa_dtype dtype, fa_mask_kind mask_kind, void* hip_stream)
{
    g_last_error[0] = '\0';
    const fa_status E = FA_ERR_INVALID_ARGUMENT;
    if (B <= 0) return fail(E, "fa_bwd: B must be > 0, got %d", B);
    if (H_q <= 0) return fail(E, "fa_bwd: H_q must be > 0, got %d", H_q);
    if (H_kv <= 0) return fail(E, "fa_bwd: H_kv must be > 0, got %d", H_kv);
    if (H_q % H_kv != 0) return fail(E, "fa_bwd: H_q (%d) must be divisible by H_kv (%d)", H_q, H_kv);
    if (qL <= 0) return fail(E, "fa_bwd: qL must be > 0, got %d", qL);
    if (kL <= 0) return fail(E, "fa_bwd: kL must be > 0, got %d", kL);
    if (D != 16 && D != 32 && D != 48 && D != 64 && D != 80 && D != 96 && D != 128 && D != 256)
        return fail(E, "fa_bwd: D must be 16, 32, 48, 64, 80, 96, 128 or 256, got %d", D);
    if (dtype != FA_DTYPE_F32 && dtype != FA_DTYPE_BF16) return fail(E, "fa_bwd: unknown dtype %d", (int)dtype);
    if (mask_kind != FA_MASK_NONE && mask_kind != FA_MASK_ADDITIVE && mask_kind != FA_MASK_BOOL)
        return fail(E, "fa_bwd: unknown mask kind %d", (int)mask_kind);
    if ((mask_kind == FA_MASK_NONE) != (mask == nullptr))
        return fail(E, "fa_bwd: mask must be NULL exactly when mask_kind is FA_MASK_NONE");
    if (!Q || !K || !V || !O || !dO || !L || !Delta || !dQ || !dK || !dV)
        return fail(E, "fa_bwd: Q, K, V, O, dO, L, Delta, dQ, dK and dV must be non-NULL");
    if (!std::isfinite(scale)) return fail(E, "fa_bwd: scale must be finite");
    if (!aligned(Q, 16) || !aligned(K, 16) || !aligned(V, 16) || !aligned(O, 16) || !aligned(dO, 16) ||
        !aligned(dQ, 16) || !aligned(dK, 16) || !aligned(dV, 16) || !aligned(L, 4) || !aligned(Delta, 4))
        return fail(E, "fa_bwd: Q, K, V, O, dO, dQ, dK and dV must be 16-byte aligned, L and Delta 4-byte aligned");
    if ((int64_t)B * H_q * qL * D > INT64_MAX / 8 || (int64_t)B * H_q * qL * kL > INT64_MAX / 8)
        return fail(E, "fa_bwd: tensor too large");
    const fa::BwdVariant* var = find_bwd_variant(dtype, D, mask_kind, causal);
    if (!var)
        return fail(FA_ERR_UNSUPPORTED, "fa_bwd: no backward kernel built for dtype %d, D %d, mask %d, causal %d "
                    "(built: bf16, D 64 and 128)", (int)dtype, D, (int)mask_kind, causal);
    fa::BwdParams p;
    std::memset(&p, 0, sizeof(p));
    p.q = Q;
    p.k = K;
    p.v = V;
    p.o = O;
    p.dout = dO;
    p.lse = L;
    p.mask = mask;
    p.delta = Delta;
    p.dq = dQ;
    p.dk = dK;
    p.dv = dV;
    default_strides(p.m_s, H_q, qL, kL);
    p.B = B;
    p.Hq = H_q;
    p.Hkv = H_kv;
    p.qL = qL;
    p.kL = kL;
    p.group = H_q / H_kv;
    p.scale = scale;
    p.scale_log2 = scale * 1.4426950408889634f;
    p.kv_split = 1;  // the dK/dV grid divides its index by it: never 0 (the launcher may raise it)
    if (mask_kind != FA_MASK_NONE) {
        const int mesz = mask_kind == FA_MASK_BOOL ? 1 : 2;
        p.mask_vec = aligned(mask, (uintptr_t)4 * mesz) && kL % 4 == 0;
    }
    const int64_t grid = std::max<int64_t>((int64_t)(qL + 127) / 128 * H_q * B, (int64_t)(kL + 127) / 128 * H_kv * B);
    if (grid > 0x7fffffffLL || (int64_t)B * H_q * qL * (D / 8) / 256 > 0x7fffffffLL)
        return fail(E, "fa_bwd: grid too large");
    const hipError_t err = var->launch(p, (hipStream_t)hip_stream);
    if (err != hipSuccess) return fail(FA_ERR_HIP, "fa_bwd: launch of %s failed: %s", var->name, hipGetErrorString(err));
    return FA_OK;
}

fa_status fa_fwd(const void* Q, const void* K, const void* V, const void* mask,
                 void* O, float* L,
                 int B, int H_q, int H_kv, int qL, int kL, int D,
                 float scale, int causal,
                 fa_dtype dtype, fa_mask_kind mask_kind, void* hip_stream)
{
    return fa_fwd_strided(Q, K, V, mask, O, L, B, H_q, H_kv, qL, kL, D, scale, causal, dtype, mask_kind,
                          nullptr, hip_stream);
}

}  // extern "C"
