// C-ABI host side: configuration checks and named refusals, arena planning,
// the kernel sequence of one micro-batch, AdamW, and exact state bytes.
//
// The sequence follows the decoder of the MojoLearn 162M model card
// (pre-norm RMSNorm, rotary attention, SwiGLU, no final norm, untied tables)
// and its "Training" table (shard gradients summed in a fixed order, AdamW with
// beta (0.9, 0.95), eps 1e-8, weight decay 0.1). The bit-level rules (MLB-P1)
// live with the kernels; the host only orders launches and never does
// arithmetic on tensor data, except the three scalars it hands to kernels:
// 1/N, the attention scale RN(1/sqrt(hd)) and the AdamW bias corrections
// RN(1 - beta^t) with beta^t a binary64 product of the binary32 beta.
#include <hip/hip_runtime.h>

#include <cmath>
#include <cstdarg>
#include <cstdio>
#include <algorithm>
#include <cstring>
#include <map>
#include <mutex>
#include <string>
#include <thread>
#include <utility>
#include <vector>

#include "../../include/mlb.h"
#include "../../include/mlb_prim.h"
#include "mlb_internal.hpp"

namespace {

thread_local char g_msg[512] = "";

mlb_status fail(mlb_status s, const char* fmt, ...) {
    va_list ap;
    va_start(ap, fmt);
    std::vsnprintf(g_msg, sizeof g_msg, fmt, ap);
    va_end(ap);
    return s;
}

#define HIPCHK(x)                                                                                \
    do {                                                                                         \
        hipError_t e_ = (x);                                                                     \
        if (e_ != hipSuccess) return fail(MLB_E_DEVICE, "%s: %s", #x, hipGetErrorString(e_)); \
    } while (0)
#define KCHK(x)                                                             \
    do {                                                                    \
        int r_ = (x);                                                       \
        if (r_ != 0) return fail(MLB_E_DEVICE, "%s returned %d", #x, r_); \
    } while (0)

// ------------------------------------------------------------------ SHA-256
// FIPS 180-4, written for this library (state bytes and their digests).
class Sha {
public:
    Sha() { reset(); }
    void reset() {
        static const uint32_t h0[8] = {0x6a09e667u, 0xbb67ae85u, 0x3c6ef372u, 0xa54ff53au,
                                       0x510e527fu, 0x9b05688cu, 0x1f83d9abu, 0x5be0cd19u};
        for (int i = 0; i < 8; ++i) st_[i] = h0[i];
        nbytes_ = 0;
        used_ = 0;
    }
    void add(const void* data, size_t n) {
        const uint8_t* p = static_cast<const uint8_t*>(data);
        nbytes_ += n;
        if (used_) {
            while (n && used_ < 64) { blk_[used_++] = *p++; --n; }
            if (used_ == 64) { compress(blk_); used_ = 0; }
        }
        while (n >= 64) { compress(p); p += 64; n -= 64; }
        while (n) { blk_[used_++] = *p++; --n; }
    }
    void digest(uint8_t out[32]) {
        const uint64_t bits = nbytes_ * 8u;
        const uint8_t one = 0x80, zero = 0;
        add(&one, 1);
        while (used_ != 56) add(&zero, 1);
        uint8_t len[8];
        for (int i = 0; i < 8; ++i) len[i] = (uint8_t)(bits >> (8 * (7 - i)));
        add(len, 8);
        for (int i = 0; i < 8; ++i)
            for (int b = 0; b < 4; ++b) out[4 * i + b] = (uint8_t)(st_[i] >> (24 - 8 * b));
    }

private:
    static uint32_t ror(uint32_t x, unsigned r) { return (x >> r) | (x << (32u - r)); }
    void compress(const uint8_t* p) {
        static const uint32_t k[64] = {
            0x428a2f98u, 0x71374491u, 0xb5c0fbcfu, 0xe9b5dba5u, 0x3956c25bu, 0x59f111f1u, 0x923f82a4u, 0xab1c5ed5u,
            0xd807aa98u, 0x12835b01u, 0x243185beu, 0x550c7dc3u, 0x72be5d74u, 0x80deb1feu, 0x9bdc06a7u, 0xc19bf174u,
            0xe49b69c1u, 0xefbe4786u, 0x0fc19dc6u, 0x240ca1ccu, 0x2de92c6fu, 0x4a7484aau, 0x5cb0a9dcu, 0x76f988dau,
            0x983e5152u, 0xa831c66du, 0xb00327c8u, 0xbf597fc7u, 0xc6e00bf3u, 0xd5a79147u, 0x06ca6351u, 0x14292967u,
            0x27b70a85u, 0x2e1b2138u, 0x4d2c6dfcu, 0x53380d13u, 0x650a7354u, 0x766a0abbu, 0x81c2c92eu, 0x92722c85u,
            0xa2bfe8a1u, 0xa81a664bu, 0xc24b8b70u, 0xc76c51a3u, 0xd192e819u, 0xd6990624u, 0xf40e3585u, 0x106aa070u,
            0x19a4c116u, 0x1e376c08u, 0x2748774cu, 0x34b0bcb5u, 0x391c0cb3u, 0x4ed8aa4au, 0x5b9cca4fu, 0x682e6ff3u,
            0x748f82eeu, 0x78a5636fu, 0x84c87814u, 0x8cc70208u, 0x90befffau, 0xa4506cebu, 0xbef9a3f7u, 0xc67178f2u};
        uint32_t w[64];
        for (int t = 0; t < 16; ++t)
            w[t] = ((uint32_t)p[4 * t] << 24) | ((uint32_t)p[4 * t + 1] << 16) | ((uint32_t)p[4 * t + 2] << 8) |
                   (uint32_t)p[4 * t + 3];
        for (int t = 16; t < 64; ++t)
            w[t] = (ror(w[t - 2], 17) ^ ror(w[t - 2], 19) ^ (w[t - 2] >> 10)) + w[t - 7] +
                   (ror(w[t - 15], 7) ^ ror(w[t - 15], 18) ^ (w[t - 15] >> 3)) + w[t - 16];
        uint32_t v[8];
        for (int i = 0; i < 8; ++i) v[i] = st_[i];
        for (int t = 0; t < 64; ++t) {
            const uint32_t t1 = v[7] + (ror(v[4], 6) ^ ror(v[4], 11) ^ ror(v[4], 25)) +
                                ((v[4] & v[5]) ^ (~v[4] & v[6])) + k[t] + w[t];
            const uint32_t t2 = (ror(v[0], 2) ^ ror(v[0], 13) ^ ror(v[0], 22)) +
                                ((v[0] & v[1]) ^ (v[0] & v[2]) ^ (v[1] & v[2]));
            for (int i = 7; i > 0; --i) v[i] = v[i - 1];
            v[4] += t1;
            v[0] = t1 + t2;
        }
        for (int i = 0; i < 8; ++i) st_[i] += v[i];
    }
    uint32_t st_[8];
    uint8_t blk_[64];
    uint64_t nbytes_;
    size_t used_;
};

void sha256_bytes(const void* p, size_t n, uint8_t out[32]) {
    Sha s;
    s.add(p, n);
    s.digest(out);
}

// ------------------------------------------------------------ layout
constexpr size_t ALIGN = 256;
constexpr int64_t KCH = 1024;
constexpr int64_t MAX_TOKENS = mlb::EMBED_MAX_POSITIONS;   // 65,536 tokens per micro-batch

struct Sizes {
    int64_t V, d, L, H, hd, F, B, T, N, P;
    int64_t ldV;   // logits row stride: V rounded up to 4 so rows take float4 loads
    bool tied;
};

bool cfg_valid(const mlb_config* c, std::string* why) {
    if (!c) { *why = "config is null"; return false; }
    if (c->abi_version != MLB_ABI_VERSION) { *why = "abi_version mismatch"; return false; }
    if (!c->vocab || !c->d_model || !c->n_layers || !c->n_heads || !c->head_dim || !c->ffn_hidden || !c->batch ||
        !c->seq_len) { *why = "zero-sized dimension"; return false; }
    if ((uint64_t)c->n_heads * c->head_dim != c->d_model) { *why = "d_model != n_heads * head_dim"; return false; }
    if (c->tied > 1) { *why = "tied must be 0 or 1"; return false; }
    const float f[6] = {c->rope_theta, c->rms_eps, c->beta1, c->beta2, c->adam_eps, c->weight_decay};
    for (float x : f)
        if (!std::isfinite(x)) { *why = "non-finite hyper-parameter"; return false; }
    return true;
}

// Shapes the kernels are not built for: a named refusal, never a slower path.
bool cfg_supported(const mlb_config* c, std::string* why) {
    if (c->head_dim % 2) { *why = "rotary pairs need an even head_dim"; return false; }
    if (c->d_model % 32 || c->ffn_hidden % 32) { *why = "d_model and ffn_hidden must be multiples of 32"; return false; }
    if (c->seq_len % 32) { *why = "seq_len must be a multiple of 32 (32x32 attention tiles)"; return false; }
    if ((uint64_t)c->batch * c->seq_len > (uint64_t)MAX_TOKENS) {
        *why = "more than 65,536 tokens per micro-batch";
        return false;
    }
    if (c->vocab > 0x7fffffffu) { *why = "vocab too large"; return false; }
    return true;
}

Sizes sizes_of(const mlb_config* c) {
    Sizes s;
    s.V = c->vocab; s.d = c->d_model; s.L = c->n_layers; s.H = c->n_heads; s.hd = c->head_dim;
    s.F = c->ffn_hidden; s.B = c->batch; s.T = c->seq_len; s.N = s.B * s.T; s.tied = c->tied != 0;
    s.ldV = (s.V + 3) / 4 * 4;
    s.P = s.V * s.d + s.L * (2 * s.d + 4 * s.d * s.d + 3 * s.F * s.d) + (s.tied ? 0 : s.V * s.d);
    return s;
}

// Arena carve-up; the same walk sizes the arena and assigns the pointers.
struct Carve {
    char* base;
    size_t off = 0;
    template <class T> T* take(int64_t n) {
        off = (off + ALIGN - 1) / ALIGN * ALIGN;
        T* p = base ? reinterpret_cast<T*>(base + off) : nullptr;
        off += (size_t)n * sizeof(T);
        return p;
    }
};

int64_t split_floats(const Sizes& s) {
    // per-chunk partials of the weight-gradient contractions over N tokens
    mlb::GemmPlan auto_plan;
    int64_t best = 0;
    // {M, N, K, kseg} of every contraction of the step
    const int64_t shapes[][4] = {{3 * s.d, s.d, s.N, s.N}, {s.d, s.d, s.N, s.N},    {2 * s.F, s.d, s.N, s.N},
                                 {s.d, s.F, s.N, s.N},     {s.V, s.d, s.N, s.N},    {s.N, s.d, s.V, s.V},
                                 {s.N, s.d, s.F, s.F},     {s.N, s.d, 2 * s.F, s.F}, {s.N, s.d, 3 * s.d, s.d},
                                 {s.N, s.F, s.d, s.d},     {s.N, s.d, s.d, s.d}};
    int64_t f[11];
    for (int i = 0; i < 11; ++i) {
        mlb::GemmDesc g;
        g.M = shapes[i][0]; g.N = shapes[i][1]; g.K = shapes[i][2]; g.kseg = shapes[i][3];
        f[i] = mlb::gemm_split_scratch(g, auto_plan);
        if (f[i] > best) best = f[i];
    }
    // the q/k/v and Wo weight gradients run as one launch (gemm_pair)
    return best > f[0] + f[1] ? best : f[0] + f[1];
}

}  // namespace

struct StatRec {
    std::string site, kernel;
    double flops = 0, bytes = 0;
    hipEvent_t e0 = nullptr, e1 = nullptr;
};
struct StatAgg {
    std::string site, kernel;
    int64_t launches = 0;
    double ms = 0, flops = 0, bytes = 0;
};

// Activation-gradient buffers shared by the caller's stream and the library's
// side stream (which runs the weight-gradient work of the backward pass). The
// main stream overwrites a slot only after the side stream's last reader of it
// has finished (per-slot event).
struct Ring {
    std::vector<float*> buf;
    std::vector<hipEvent_t> ev;
    std::vector<char> pending;
};

struct mlb_model {
    mlb_config cfg;
    Sizes s;
    hipStream_t stream;        // the caller's stream: every call is ordered on it
    hipStream_t side = nullptr;
    hipStream_t cur = nullptr; // the stream the op being enqueued runs on
    hipEvent_t sorted = nullptr;   // the embedding keys of the last training forward are sorted (side stream)
    bool overlap = false;      // backward weight-gradient work on the side stream (off: one stream is faster)
    std::vector<hipEvent_t> sync_pool;
    size_t sync_next = 0;
    int device;
    // parameter offsets (floats)
    int64_t offE, offOut;
    std::vector<int64_t> o_w1, o_qkv, o_wo, o_w2, o_gu, o_wd;
    // state
    float *p, *G, *m, *v;
    float *cosv, *sinv;
    int32_t *ids, *tg;
    int* err;
    float* loss_dev;
    float* loss_rows;
    std::vector<float*> h, xn1, r1, qkv, P, O, hmid, xn2, r2, gu, a;   // h has L+1 entries
    float* logits;
    Ring dh, dgu, dxn, dqkv;
    float *dA, *dO, *dP, *Dv, *gE, *split, *split_side, *dwpart;
    int64_t* dw_offs;   // the norm gains' offsets in G, in the order of their partial slots
    int64_t split_n;
    uint64_t* keys;
    float* host_stage;   // pinned, 64 bytes
    uint64_t step;
    bool have_fwd;
    int n_accum;
    float attn_scale, invN;
    bool stats_on = false;
    std::vector<std::string> stats_sites;   // empty: every call site is timed
    std::vector<StatRec> pending;
    std::vector<hipEvent_t> free_events;
    std::map<std::string, StatAgg> agg;
};

namespace {

// The side stream (default priority, not synchronising with the null stream),
// the pool of ordering events and one event per ring slot.
mlb_status make_streams(mlb_model* M) {
    if (hipStreamCreateWithFlags(&M->side, hipStreamNonBlocking) != hipSuccess)
        return fail(MLB_E_DEVICE, "side stream");
    if (hipEventCreateWithFlags(&M->sorted, hipEventDisableTiming) != hipSuccess) return fail(MLB_E_DEVICE, "event");
    M->sync_pool.assign(64, nullptr);
    for (hipEvent_t& e : M->sync_pool)
        if (hipEventCreateWithFlags(&e, hipEventDisableTiming) != hipSuccess) return fail(MLB_E_DEVICE, "event");
    for (Ring* r : {&M->dh, &M->dgu, &M->dxn, &M->dqkv}) {
        r->ev.assign(r->buf.size(), nullptr);
        r->pending.assign(r->buf.size(), 0);
        for (hipEvent_t& e : r->ev)
            if (hipEventCreateWithFlags(&e, hipEventDisableTiming) != hipSuccess) return fail(MLB_E_DEVICE, "event");
    }
    M->cur = M->stream;
    return MLB_OK;
}

void release_streams(mlb_model* M) {
    if (M->side) (void)hipStreamSynchronize(M->side);
    for (hipEvent_t e : M->sync_pool)
        if (e) (void)hipEventDestroy(e);
    for (Ring* r : {&M->dh, &M->dgu, &M->dxn, &M->dqkv})
        for (hipEvent_t e : r->ev)
            if (e) (void)hipEventDestroy(e);
    if (M->sorted) (void)hipEventDestroy(M->sorted);
    M->sorted = nullptr;
    if (M->side) (void)hipStreamDestroy(M->side);
    M->side = nullptr;
    M->sync_pool.clear();
}

size_t carve(mlb_model* M, char* base) {
    const Sizes& s = M->s;
    Carve c{base};
    M->p = c.take<float>(s.P);
    M->G = c.take<float>(s.P);
    M->m = c.take<float>(s.P);
    M->v = c.take<float>(s.P);
    M->cosv = c.take<float>(s.T * s.hd / 2);
    M->sinv = c.take<float>(s.T * s.hd / 2);
    M->ids = c.take<int32_t>(s.N);
    M->tg = c.take<int32_t>(s.N);
    M->err = c.take<int>(64);
    M->loss_dev = c.take<float>(64);
    M->loss_rows = c.take<float>(s.N);
    M->h.assign(s.L + 1, nullptr);
    for (auto* vec : {&M->xn1, &M->r1, &M->qkv, &M->P, &M->O, &M->hmid, &M->xn2, &M->r2, &M->gu, &M->a})
        vec->assign(s.L, nullptr);
    for (int64_t l = 0; l <= s.L; ++l) M->h[l] = c.take<float>(s.N * s.d);
    for (int64_t l = 0; l < s.L; ++l) {
        M->xn1[l] = c.take<float>(s.N * s.d);
        M->r1[l] = c.take<float>(s.N);
        M->qkv[l] = c.take<float>(s.N * 3 * s.d);
        M->P[l] = c.take<float>(s.B * s.H * s.T * s.T);
        M->O[l] = c.take<float>(s.N * s.d);
        M->hmid[l] = c.take<float>(s.N * s.d);
        M->xn2[l] = c.take<float>(s.N * s.d);
        M->r2[l] = c.take<float>(s.N);
        M->gu[l] = c.take<float>(s.N * 2 * s.F);
        M->a[l] = c.take<float>(s.N * s.F);
    }
    M->logits = c.take<float>(s.N * s.ldV);
    auto ring = [&](Ring& r, int n, int64_t floats) {
        r.buf.resize(n);
        for (int i = 0; i < n; ++i) r.buf[i] = c.take<float>(floats);
    };
    ring(M->dh, 4, s.N * s.d);
    M->dA = c.take<float>(s.N * s.F);
    ring(M->dgu, 2, s.N * 2 * s.F);
    ring(M->dxn, 4, s.N * s.d);
    M->dO = c.take<float>(s.N * s.d);
    ring(M->dqkv, 2, s.N * 3 * s.d);
    M->dP = c.take<float>(s.B * s.H * s.T * s.T);
    M->Dv = c.take<float>(s.B * s.H * s.T);
    M->gE = s.tied ? c.take<float>(s.V * s.d) : nullptr;
    M->split_n = split_floats(s);
    M->split = c.take<float>(M->split_n > 0 ? M->split_n : 1);
    M->split_side = c.take<float>(M->split_n > 0 ? M->split_n : 1);
    // every norm gain's chunk partials of one micro-batch (two per layer), folded
    // into G together at the end of the backward
    M->dwpart = c.take<float>(2 * s.L * ((s.N + KCH - 1) / KCH) * s.d);
    M->dw_offs = c.take<int64_t>(2 * s.L);
    M->keys = c.take<uint64_t>(mlb::embed_key_slots(s.N));
    return c.off + ALIGN;
}

void offsets(mlb_model* M) {
    const Sizes& s = M->s;
    int64_t o = 0;
    M->offE = o; o += s.V * s.d;
    for (int64_t l = 0; l < s.L; ++l) {
        M->o_w1.push_back(o); o += s.d;
        M->o_qkv.push_back(o); o += 3 * s.d * s.d;
        M->o_wo.push_back(o); o += s.d * s.d;
        M->o_w2.push_back(o); o += s.d;
        M->o_gu.push_back(o); o += 2 * s.F * s.d;
        M->o_wd.push_back(o); o += s.d * s.F;
    }
    M->offOut = s.tied ? M->offE : o;
}

// Step-0 parameters from a seed (callers that pass none). SplitMix64 in its
// counter form: output i is the variant-13 finaliser applied to seed + (i + 1)
// * 0x9E3779B97F4A7C15. Parameter k takes outputs 2k and 2k+1 through the
// Box-Muller transform in binary64; norm gains are 1 + 0.02 z, the rest 0.02 z,
// rounded once. Host threads split the index range (each value depends on k
// only).
uint64_t splitmix_at(uint64_t seed, uint64_t i) {
    uint64_t z = seed + (i + 1) * 0x9E3779B97F4A7C15ull;
    z = (z ^ (z >> 30)) * 0xBF58476D1CE4E5B9ull;
    z = (z ^ (z >> 27)) * 0x94D049BB133111EBull;
    return z ^ (z >> 31);
}

std::vector<float> seeded_params(const mlb_model* M, uint64_t seed) {
    const Sizes& s = M->s;
    std::vector<float> out((size_t)s.P);
    std::vector<char> gain((size_t)s.P, 0);
    for (int64_t l = 0; l < s.L; ++l)
        for (int64_t c = 0; c < s.d; ++c) gain[(size_t)(M->o_w1[l] + c)] = gain[(size_t)(M->o_w2[l] + c)] = 1;
    auto fill = [&](int64_t lo, int64_t hi) {
        for (int64_t k = lo; k < hi; ++k) {
            const uint64_t r1 = splitmix_at(seed, 2 * (uint64_t)k), r2 = splitmix_at(seed, 2 * (uint64_t)k + 1);
            const double u1 = (double)((r1 >> 11) + 1) * 0x1p-53;
            const double u2 = (double)(r2 >> 11) * 0x1p-53;
            const double z = std::sqrt(-2.0 * std::log(u1)) * std::cos(6.283185307179586 * u2);
            const double w = 0.02 * z;
            out[(size_t)k] = gain[(size_t)k] ? (float)(1.0 + w) : (float)w;
        }
    };
    const int64_t nthr = 8, per = (s.P + nthr - 1) / nthr;
    std::vector<std::thread> th;
    for (int64_t t = 0; t < nthr; ++t) th.emplace_back(fill, t * per, std::min(s.P, (t + 1) * per));
    for (auto& x : th) x.join();
    return out;
}

// RoPE table: cos/sin of t * theta^(-2i/hd), binary64 on the host, rounded.
void rope_table_host(int64_t T, int64_t hd, float theta, std::vector<float>& c, std::vector<float>& sn) {
    const int64_t h2 = hd / 2;
    c.resize(T * h2);
    sn.resize(T * h2);
    for (int64_t t = 0; t < T; ++t)
        for (int64_t i = 0; i < h2; ++i) {
            const double ex = -(2.0 * (double)i) / (double)hd;
            const double ang = (double)t * std::pow((double)theta, ex);
            c[t * h2 + i] = (float)std::cos(ang);
            sn[t * h2 + i] = (float)std::sin(ang);
        }
}

float bias_corr(float beta, uint64_t t) {
    double b = 1.0;
    for (uint64_t i = 0; i < t; ++i) b *= (double)beta;
    return (float)(1.0 - b);
}

mlb::GemmDesc lin(int64_t M, int64_t N, int64_t K, const float* A, int64_t lda, bool akc, const float* B,
                  int64_t ldb, bool bkc, float* C, int64_t ldc, int mode) {
    mlb::GemmDesc g;
    g.M = M; g.N = N; g.K = K; g.kseg = K;
    g.A = A; g.lda = lda; g.a_kc = akc;
    g.B = B; g.ldb = ldb; g.b_kc = bkc;
    g.C = C; g.ldc = ldc; g.mode = mode;
    return g;
}

// ------------------------------------------------------------ launch stats
// Optional per-launch timing with HIP events on the stream the launch runs on
// (the caller's or the side stream), grouped by call site, with each launch's algorithmic work (FLOPs of the contraction's
// valid pairs, or the minimal HBM bytes of a row/elementwise kernel).
int64_t stat_begin(mlb_model* M, const char* site) {
    if (!M->stats_on) return -1;
    if (!M->stats_sites.empty() &&
        std::find(M->stats_sites.begin(), M->stats_sites.end(), site) == M->stats_sites.end())
        return -1;
    hipEvent_t e0 = nullptr, e1 = nullptr;
    if (M->free_events.size() >= 2) {
        e0 = M->free_events.back(); M->free_events.pop_back();
        e1 = M->free_events.back(); M->free_events.pop_back();
    } else {
        if (hipEventCreate(&e0) != hipSuccess || hipEventCreate(&e1) != hipSuccess) return -1;
    }
    if (hipEventRecord(e0, M->cur) != hipSuccess) return -1;
    StatRec r;
    r.e0 = e0; r.e1 = e1;
    M->pending.push_back(r);
    return (int64_t)M->pending.size() - 1;
}

void stat_end(mlb_model* M, int64_t idx, const char* site, const char* kernel, double flops, double bytes) {
    if (idx < 0) return;
    StatRec& r = M->pending[(size_t)idx];
    (void)hipEventRecord(r.e1, M->cur);
    r.site = site; r.kernel = kernel; r.flops = flops; r.bytes = bytes;
}

// Call only after the stream is synchronised.
void stat_resolve(mlb_model* M) {
    for (StatRec& r : M->pending) {
        float ms = 0.0f;
        if (hipEventElapsedTime(&ms, r.e0, r.e1) != hipSuccess) ms = 0.0f;
        StatAgg& a = M->agg[r.site + "|" + r.kernel];
        a.site = r.site; a.kernel = r.kernel;
        a.launches += 1; a.ms += ms; a.flops += r.flops; a.bytes += r.bytes;
        M->free_events.push_back(r.e0);
        M->free_events.push_back(r.e1);
    }
    M->pending.clear();
}

// Every dispatch of a contraction is timed on its own, with its own FLOPs.
struct GemmStatCtx {
    mlb_model* M;
    const char* site;
    int64_t ev;
};
void gemm_stat_begin(void* c) {
    auto* x = static_cast<GemmStatCtx*>(c);
    x->ev = stat_begin(x->M, x->site);
}
void gemm_stat_end(void* c, const char* kernel, double flops, double bytes) {
    auto* x = static_cast<GemmStatCtx*>(c);
    stat_end(x->M, x->ev, x->site, kernel, flops, bytes);
}

mlb_status run_gemm(mlb_model* M, const char* site, const mlb::GemmDesc& g) {
    mlb::GemmPlan p;
    p.scratch = (M->overlap && M->cur == M->side) ? M->split_side : M->split;   // one split scratch per stream
    p.scratch_floats = M->split_n;
    GemmStatCtx ctx{M, site, -1};
    mlb::LaunchTrace tr;
    tr.ctx = &ctx; tr.begin = gemm_stat_begin; tr.end = gemm_stat_end;
    const int r = mlb::gemm(g, p, M->cur, M->stats_on ? &tr : nullptr);
    if (r != 0) return fail(MLB_E_DEVICE, "contraction %ldx%ldx%ld failed (%d)", (long)g.M, (long)g.N, (long)g.K, r);
    return MLB_OK;
}

#define RUN(site, g)                                 \
    do {                                             \
        mlb_status st_ = run_gemm(M, site, (g));     \
        if (st_ != MLB_OK) return st_;               \
    } while (0)

// Two independent contractions in one launch where they fit (mlb::gemm_pair).
mlb_status run_gemm_pair(mlb_model* M, const char* site, const mlb::GemmDesc& g0, const mlb::GemmDesc& g1) {
    mlb::GemmPlan p;
    p.scratch = (M->overlap && M->cur == M->side) ? M->split_side : M->split;
    p.scratch_floats = M->split_n;
    GemmStatCtx ctx{M, site, -1};
    mlb::LaunchTrace tr;
    tr.ctx = &ctx; tr.begin = gemm_stat_begin; tr.end = gemm_stat_end;
    const int r = mlb::gemm_pair(g0, g1, p, M->cur, M->stats_on ? &tr : nullptr);
    if (r != 0) return fail(MLB_E_DEVICE, "contraction pair %ldx%ld and %ldx%ld failed (%d)", (long)g0.M, (long)g0.N,
                            (long)g1.M, (long)g1.N, r);
    return MLB_OK;
}

// A row or elementwise kernel with its algorithmic HBM bytes.
#define OP(site, bytes, x)                                                           \
    do {                                                                             \
        const int64_t ev_ = stat_begin(M, site);                                     \
        const int r_ = (x);                                                          \
        stat_end(M, ev_, site, site, 0.0, (double)(bytes));                          \
        if (r_ != 0) return fail(MLB_E_DEVICE, "%s returned %d", #x, r_);            \
    } while (0)

// Lower-triangle contraction over the head dimension for all B*H heads:
// rows of A and B at stride ld (head h at column h*hd, batch b at b*sb).
// P and D non-null: the softmax backward runs in the epilogue (C = dS).
mlb_status run_tri(mlb_model* M, const char* site, int64_t T, int64_t hd, const float* A, int64_t lda, int64_t sAb,
                   const float* B, int64_t ldb, int64_t sBb, float* C, int scaled, float scale,
                   const float* P = nullptr, const float* D = nullptr, float ds_scale = 0.0f) {
    const Sizes& s = M->s;
    const int64_t ev = stat_begin(M, site);
    const int r = mlb::tri_nt(T, hd, s.B * s.H, s.H, A, lda, sAb, hd, B, ldb, sBb, hd, C, T, s.H * T * T, T * T,
                              scaled, scale, 1, P, D, ds_scale, M->cur);
    stat_end(M, ev, site, "k_tri_nt", 2.0 * (double)(s.B * s.H) * (double)T * (double)(T + 1) / 2.0 * (double)hd,
             0.0);
    if (r != 0) return fail(MLB_E_DEVICE, "%s failed (%d)", site, r);
    return MLB_OK;
}

// The row-strip kernel for 64-wide heads: the scores (P == nullptr), or dS
// together with dQ. Returns MLB_E_UNSUPPORTED without launching when the
// shape is not one it runs.
mlb_status run_rows(mlb_model* M, const char* site, const float* X, int64_t ldx, const float* Y, int64_t ldy,
                    float* S, float scale, const float* P = nullptr, const float* D = nullptr,
                    const float* K = nullptr, int64_t ldk = 0, float* dQ = nullptr, int64_t ldq = 0) {
    const Sizes& s = M->s;
    const int64_t T = s.T, hd = s.hd;
    if (!mlb::attn_rows_fits(T, hd, s.B * s.H, s.H, X, ldx, T * ldx, hd, Y, ldy, T * ldy, hd, S, T, s.H * T * T,
                             T * T))
        return MLB_E_UNSUPPORTED;
    const double tri = 2.0 * (double)(s.B * s.H) * (double)T * (double)(T + 1) / 2.0 * (double)hd;
    const int64_t ev = stat_begin(M, site);
    const int r = mlb::attn_rows(T, hd, s.B * s.H, s.H, X, ldx, T * ldx, hd, Y, ldy, T * ldy, hd, S, T, s.H * T * T,
                                 T * T, scale, P, D, K, ldk, T * ldk, hd, dQ, ldq, T * ldq, hd, M->cur);
    stat_end(M, ev, site, P ? "k_attn_rows<dS,dQ>" : "k_attn_rows<S>", P ? 2.0 * tri : tri, 0.0);
    if (r != 0) return fail(MLB_E_DEVICE, "%s failed (%d)", site, r);
    return MLB_OK;
}

#define TRI(site, ...)                                       \
    do {                                                     \
        mlb_status st_ = run_tri(M, site, __VA_ARGS__);      \
        if (st_ != MLB_OK) return st_;                       \
    } while (0)

// Per-head attention contractions on [N, 3d] (q | k | v) and [N, d] rows.
mlb::GemmDesc head_gemm(const Sizes& s) {
    mlb::GemmDesc g;
    g.batch = s.B * s.H;
    g.H = s.H;
    return g;
}

// mode 0: training (loss, d-logits in place of the logits); 1: inference with
// loss (the logits are kept); 2: inference, logits only.
mlb_status stream_wait(mlb_model* M, hipStream_t from, hipStream_t to);

mlb_status forward(mlb_model* M, int mode = 0) {
    const Sizes& s = M->s;
    hipStream_t st = M->stream;
    M->cur = st;
    const int64_t N = s.N, d = s.d, F = s.F, T = s.T, H = s.H, hd = s.hd, BH = s.B * s.H;
    const double f4 = 4.0, tri = (double)BH * (double)T * (double)(T + 1) / 2.0;
    OP("embed_gather", f4 * 2 * N * d, mlb::gather_rows(M->ids, M->p + M->offE, s.V, d, N, M->h[0], M->err, st));
    if (mode == 0) {
        // the embedding gradient's key sort needs the ids only: it runs on the
        // side stream beside the forward and is joined by the backward's scatter
        const mlb_status ws = stream_wait(M, st, M->side);
        if (ws != MLB_OK) return ws;
        M->cur = M->side;
        OP("embed_sort", f4 * N, mlb::embed_sort(M->ids, N, s.V, M->keys, M->side));
        if (hipEventRecord(M->sorted, M->side) != hipSuccess) return fail(MLB_E_DEVICE, "sort event");
        M->cur = st;
    }
    for (int64_t l = 0; l < s.L; ++l) {
        OP("rmsnorm_fwd", f4 * (2 * N * d + N + d),
           mlb::rmsnorm_fwd(M->h[l], M->p + M->o_w1[l], N, d, M->cfg.rms_eps, M->xn1[l], M->r1[l], st));
        mlb::GemmDesc qkv = lin(N, 3 * d, d, M->xn1[l], d, true, M->p + M->o_qkv[l], d, true, M->qkv[l], 3 * d, 0);
        if (hd == 64) {   // q and k rotated in the contraction's epilogue
            qkv.rope_cos = M->cosv; qkv.rope_sin = M->sinv; qkv.rope_T = T; qkv.rope_cols = 2 * d;
        }
        RUN("qkv_fwd", qkv);
        if (hd != 64) {
            OP("rope_fwd", f4 * 2 * N * d, mlb::rope(M->qkv[l], s.B, T, H, hd, 3 * d, M->cosv, M->sinv, 0, st));
            OP("rope_fwd", f4 * 2 * N * d, mlb::rope(M->qkv[l] + d, s.B, T, H, hd, 3 * d, M->cosv, M->sinv, 0, st));
        }
        // S = (q . k) * scale, j <= i
        const mlb_status sr = run_rows(M, "attn_scores", M->qkv[l], 3 * d, M->qkv[l] + d, 3 * d, M->P[l],
                                       M->attn_scale);
        if (sr == MLB_E_UNSUPPORTED)
            TRI("attn_scores", T, hd, M->qkv[l], 3 * d, T * 3 * d, M->qkv[l] + d, 3 * d, T * 3 * d, M->P[l], 1,
                M->attn_scale);
        else if (sr != MLB_OK) return sr;
        OP("softmax_fwd", f4 * 2 * tri, mlb::softmax_causal(M->P[l], BH, T, 1, st));
        mlb::GemmDesc pv = head_gemm(s);   // O = P v over j <= i
        pv.M = T; pv.N = hd; pv.K = T; pv.kseg = T; pv.a_blk = true; pv.krange = 1;
        pv.A = M->P[l]; pv.lda = T; pv.a_kc = true; pv.sAb = H * T * T; pv.sAh = T * T;
        pv.B = M->qkv[l] + 2 * d; pv.ldb = 3 * d; pv.b_kc = false; pv.sBb = T * 3 * d; pv.sBh = hd;
        pv.C = M->O[l]; pv.ldc = d; pv.sCb = T * d; pv.sCh = hd;
        RUN("attn_pv", pv);
        mlb::GemmDesc wo = lin(N, d, d, M->O[l], d, true, M->p + M->o_wo[l], d, true, M->hmid[l], d, 3);
        wo.R = M->h[l];                    // hmid = h + O Wo^T
        RUN("wo_fwd", wo);
        OP("rmsnorm_fwd", f4 * (2 * N * d + N + d),
           mlb::rmsnorm_fwd(M->hmid[l], M->p + M->o_w2[l], N, d, M->cfg.rms_eps, M->xn2[l], M->r2[l], st));
        RUN("gu_fwd", lin(N, 2 * F, d, M->xn2[l], d, true, M->p + M->o_gu[l], d, true, M->gu[l], 2 * F, 0));
        OP("swiglu_fwd", f4 * 3 * N * F, mlb::swiglu_fwd(M->gu[l], N, F, M->a[l], st));
        mlb::GemmDesc wd = lin(N, d, F, M->a[l], F, true, M->p + M->o_wd[l], F, true, M->h[l + 1], d, 3);
        wd.R = M->hmid[l];                 // h' = hmid + a Wd^T
        RUN("down_fwd", wd);
    }
    RUN("head_fwd", lin(N, s.V, d, M->h[s.L], d, true, M->p + M->offOut, d, true, M->logits, s.ldV, 0));
    if (mode == 2) return MLB_OK;
    OP("xent", f4 * (mode == 0 ? 2 : 1) * N * s.V,
       mlb::cross_entropy(M->logits, M->tg, N, s.V, s.ldV, M->loss_rows, mode == 0 ? M->logits : nullptr, M->err,
                          st));
    OP("loss_sum", f4 * N, mlb::sum64_scaled(M->loss_rows, N, M->invN, M->loss_dev, st));
    return MLB_OK;
}

// Cross-stream ordering: `to` waits for everything enqueued on `from` so far.
mlb_status stream_wait(mlb_model* M, hipStream_t from, hipStream_t to) {
    hipEvent_t e = M->sync_pool[M->sync_next];
    M->sync_next = (M->sync_next + 1) % M->sync_pool.size();
    if (hipEventRecord(e, from) != hipSuccess || hipStreamWaitEvent(to, e, 0) != hipSuccess)
        return fail(MLB_E_DEVICE, "stream ordering event");
    return MLB_OK;
}

// The caller's stream is about to overwrite slot k of a ring.
mlb_status ring_claim(mlb_model* M, Ring& r, int k) {
    if (r.pending[k]) {
        if (hipStreamWaitEvent(M->stream, r.ev[k], 0) != hipSuccess) return fail(MLB_E_DEVICE, "ring wait");
        r.pending[k] = 0;
    }
    return MLB_OK;
}

// The side stream has enqueued its (last) reader of slot k.
mlb_status ring_read(mlb_model* M, Ring& r, int k) {
    if (!M->overlap) return MLB_OK;   // one stream: program order suffices
    if (hipEventRecord(r.ev[k], M->side) != hipSuccess) return fail(MLB_E_DEVICE, "ring event");
    r.pending[k] = 1;
    return MLB_OK;
}

#define CHK(x)                                  \
    do {                                        \
        mlb_status st_ = (x);                   \
        if (st_ != MLB_OK) return st_;          \
    } while (0)

// The backward pass runs on two streams. The caller's stream carries the
// chain that produces each layer's input gradient; the side stream carries
// the work that only feeds the gradient accumulator G (the weight-gradient
// contractions, the norm gains, the embedding scatter), each started once its
// inputs exist. Each G entry still receives exactly one addition per
// micro-batch, in call order (one side stream), so the bits do not depend on
// how the two streams interleave. The side stream joins the caller's stream at
// the end.
// Partial slot k of the norm gains' chunk partials (k = 2l: the MLP norm of
// layer l, 2l + 1: its attention norm).
static float* dw_slot(mlb_model* M, int64_t k) {
    return M->dwpart + k * ((M->s.N + KCH - 1) / KCH) * M->s.d;
}

mlb_status backward(mlb_model* M) {
    const Sizes& s = M->s;
    const bool two = M->overlap;
    hipStream_t st = M->stream, ss = two ? M->side : M->stream;
    const int64_t N = s.N, d = s.d, F = s.F, T = s.T, H = s.H, hd = s.hd, BH = s.B * s.H;
    const double f4 = 4.0;
    const float* dl = M->logits;
    auto on_main = [&]() { M->cur = st; };
    auto to_side = [&]() -> mlb_status {   // the side stream sees everything the main stream did so far
        M->cur = ss;
        return two ? stream_wait(M, st, ss) : MLB_OK;
    };
    Ring &DH = M->dh, &DGU = M->dgu, &DXN = M->dxn, &DQKV = M->dqkv;

    // head: dh = dl W_out (K = V); W_out gradient = dl^T h_L (K = N)
    CHK(to_side());
    if (s.tied) RUN("head_dw", lin(s.V, d, N, dl, s.ldV, false, M->h[s.L], d, false, M->gE, d, 0));
    else RUN("head_dw", lin(s.V, d, N, dl, s.ldV, false, M->h[s.L], d, false, M->G + M->offOut, d, 1));
    on_main();
    int kh = 0;
    CHK(ring_claim(M, DH, kh));
    RUN("head_dx", lin(N, d, s.V, dl, s.ldV, true, M->p + M->offOut, d, false, DH.buf[kh], d, 0));
    for (int64_t l = s.L - 1; l >= 0; --l) {
        const int kg = (int)(l % 2), kx2 = (int)(2 * (l % 2)), kx1 = kx2 + 1, kq = (int)(l % 2);
        float* dh0 = DH.buf[kh];
        // MLP branch
        RUN("down_dx", lin(N, F, d, dh0, d, true, M->p + M->o_wd[l], F, false, M->dA, F, 0));
        CHK(to_side());
        RUN("down_dw", lin(d, F, N, dh0, d, false, M->a[l], F, false, M->G + M->o_wd[l], F, 1));
        CHK(ring_read(M, DH, kh));
        on_main();
        CHK(ring_claim(M, DGU, kg));
        OP("swiglu_bwd", f4 * 5 * N * F, mlb::swiglu_bwd(M->dA, M->gu[l], N, F, DGU.buf[kg], st));
        CHK(to_side());
        RUN("gu_dw", lin(2 * F, d, N, DGU.buf[kg], 2 * F, false, M->xn2[l], d, false, M->G + M->o_gu[l], d, 1));
        CHK(ring_read(M, DGU, kg));
        on_main();
        CHK(ring_claim(M, DXN, kx2));
        mlb::GemmDesc x2 = lin(N, d, 2 * F, DGU.buf[kg], 2 * F, true, M->p + M->o_gu[l], d, false, DXN.buf[kx2], d, 0);
        x2.kseg = F;                       // segments [dg Wg, du Wu]
        RUN("gu_dx", x2);
        CHK(to_side());
        OP("rmsnorm_dw", f4 * (2 * N * d + N + d),
           mlb::rmsnorm_bwd_dw_parts(DXN.buf[kx2], M->hmid[l], M->r2[l], N, d, dw_slot(M, 2 * l), ss));
        CHK(ring_read(M, DXN, kx2));
        on_main();
        const int kh1 = (kh + 1) % 4;
        CHK(ring_claim(M, DH, kh1));
        float* dh1 = DH.buf[kh1];
        OP("rmsnorm_dx", f4 * (4 * N * d + N + d),
           mlb::rmsnorm_bwd_dx(DXN.buf[kx2], M->hmid[l], M->p + M->o_w2[l], M->r2[l], N, d, dh0, dh1, st));
        // attention branch (its Wo weight gradient runs with the q/k/v one below)
        RUN("wo_dx", lin(N, d, d, dh1, d, true, M->p + M->o_wo[l], d, false, M->dO, d, 0));
        OP("attn_rowdot", f4 * (2 * N * d + BH * T), mlb::attn_rowdot(M->dO, M->O[l], s.B, H, T, hd, d, M->Dv, st));
        CHK(ring_claim(M, DQKV, kq));
        float* dqkv = DQKV.buf[kq];
        // dS = (P * (dO . v - D)) * scale, j <= i (dP never reaches memory);
        // with 64-wide heads dQ = dS k in the same pass
        const mlb_status dr = run_rows(M, "attn_ds_dq", M->dO, d, M->qkv[l] + 2 * d, 3 * d, M->dP, M->attn_scale,
                                       M->P[l], M->Dv, M->qkv[l] + d, 3 * d, dqkv, 3 * d);
        if (dr == MLB_E_UNSUPPORTED)
            TRI("attn_dp", T, hd, M->dO, d, T * d, M->qkv[l] + 2 * d, 3 * d, T * 3 * d, M->dP, 0, 1.0f, M->P[l],
                M->Dv, M->attn_scale);
        else if (dr != MLB_OK) return dr;
        mlb::GemmDesc dv = head_gemm(s);   // dv = P^T dO over i >= j
        dv.M = T; dv.N = hd; dv.K = T; dv.kseg = T; dv.a_blk = true; dv.krange = 2;
        dv.A = M->P[l]; dv.lda = T; dv.a_kc = false; dv.sAb = H * T * T; dv.sAh = T * T;
        dv.B = M->dO; dv.ldb = d; dv.b_kc = false; dv.sBb = T * d; dv.sBh = hd;
        dv.C = dqkv + 2 * d; dv.ldc = 3 * d; dv.sCb = T * 3 * d; dv.sCh = hd;
        RUN("attn_dv", dv);
        mlb::GemmDesc dq = head_gemm(s);   // dq = dS k over j <= i
        dq.M = T; dq.N = hd; dq.K = T; dq.kseg = T; dq.a_blk = true; dq.krange = 1;
        dq.A = M->dP; dq.lda = T; dq.a_kc = true; dq.sAb = H * T * T; dq.sAh = T * T;
        dq.B = M->qkv[l] + d; dq.ldb = 3 * d; dq.b_kc = false; dq.sBb = T * 3 * d; dq.sBh = hd;
        dq.C = dqkv; dq.ldc = 3 * d; dq.sCb = T * 3 * d; dq.sCh = hd;
        if (dr == MLB_E_UNSUPPORTED) RUN("attn_dq", dq);
        mlb::GemmDesc dk = head_gemm(s);   // dk = dS^T q over i >= j
        dk.M = T; dk.N = hd; dk.K = T; dk.kseg = T; dk.a_blk = true; dk.krange = 2;
        dk.A = M->dP; dk.lda = T; dk.a_kc = false; dk.sAb = H * T * T; dk.sAh = T * T;
        dk.B = M->qkv[l]; dk.ldb = 3 * d; dk.b_kc = false; dk.sBb = T * 3 * d; dk.sBh = hd;
        dk.C = dqkv + d; dk.ldc = 3 * d; dk.sCb = T * 3 * d; dk.sCh = hd;
        // the paired-tile kernel rotates dk back in its epilogue
        const bool dk_rope = mlb::attn_av_fits(T, hd, BH, H, M->dP, T, H * T * T, T * T, M->qkv[l], 3 * d, T * 3 * d, hd);
        if (dk_rope) { dk.rope_cos = M->cosv; dk.rope_sin = M->sinv; }
        RUN("attn_dk", dk);
        OP("rope_bwd", f4 * 2 * N * d, mlb::rope(dqkv, s.B, T, H, hd, 3 * d, M->cosv, M->sinv, 1, st));
        if (!dk_rope)
            OP("rope_bwd", f4 * 2 * N * d, mlb::rope(dqkv + d, s.B, T, H, hd, 3 * d, M->cosv, M->sinv, 1, st));
        // the q/k/v and Wo weight gradients, one launch: the Wo grid fills the
        // part-filled last wave of the q/k/v grid (disjoint parts of G, so the
        // launch order does not matter to the bits)
        CHK(to_side());
        {
            const mlb_status st_ = run_gemm_pair(
                M, "qkv_wo_dw", lin(3 * d, d, N, dqkv, 3 * d, false, M->xn1[l], d, false, M->G + M->o_qkv[l], d, 1),
                lin(d, d, N, dh1, d, false, M->O[l], d, false, M->G + M->o_wo[l], d, 1));
            if (st_ != MLB_OK) return st_;
        }
        CHK(ring_read(M, DQKV, kq));
        CHK(ring_read(M, DH, kh1));
        on_main();
        CHK(ring_claim(M, DXN, kx1));
        mlb::GemmDesc x1 = lin(N, d, 3 * d, dqkv, 3 * d, true, M->p + M->o_qkv[l], d, false, DXN.buf[kx1], d, 0);
        x1.kseg = d;                       // segments [dq Wq, dk Wk, dv Wv]
        RUN("qkv_dx", x1);
        CHK(to_side());
        OP("rmsnorm_dw", f4 * (2 * N * d + N + d),
           mlb::rmsnorm_bwd_dw_parts(DXN.buf[kx1], M->h[l], M->r1[l], N, d, dw_slot(M, 2 * l + 1), ss));
        CHK(ring_read(M, DXN, kx1));
        on_main();
        const int kh2 = (kh1 + 1) % 4;
        CHK(ring_claim(M, DH, kh2));
        OP("rmsnorm_dx", f4 * (4 * N * d + N + d),
           mlb::rmsnorm_bwd_dx(DXN.buf[kx1], M->h[l], M->p + M->o_w1[l], M->r1[l], N, d, dh1, DH.buf[kh2], st));
        kh = kh2;
    }
    // embedding rows in token order (tied: on top of the head gradient, then folded)
    CHK(to_side());
    if (hipStreamWaitEvent(ss, M->sorted, 0) != hipSuccess) return fail(MLB_E_DEVICE, "sort wait");
    if (s.tied) {
        OP("embed_scatter", f4 * 3 * N * d,
           mlb::embed_scatter_sorted(M->keys, DH.buf[kh], N, d, s.V, M->gE, M->gE, 0, ss));
        OP("embed_fold", f4 * 3 * s.V * d, mlb::add_inplace(M->G + M->offE, M->gE, s.V * d, ss));
    } else {
        OP("embed_scatter", f4 * 3 * N * d,
           mlb::embed_scatter_sorted(M->keys, DH.buf[kh], N, d, s.V, nullptr, M->G + M->offE, 1, ss));
    }
    // the norm gains: each micro-batch's chunk partials folded in chunk order
    // and added to G (each gain's slice of G takes no other update)
    OP("rmsnorm_dw_fold", f4 * (2 * s.L) * d * ((N + KCH - 1) / KCH + 2),
       mlb::fold_cols_batched(M->dwpart, N, d, 2 * s.L, M->dw_offs, M->G, ss));
    // join: the caller's stream continues after all side work
    on_main();
    if (two) CHK(stream_wait(M, ss, st));
    for (Ring* r : {&DH, &DGU, &DXN, &DQKV}) std::fill(r->pending.begin(), r->pending.end(), 0);
    return MLB_OK;
}

}  // namespace

extern "C" {

int64_t mlb_param_count(const mlb_config* cfg) {
    std::string why;
    if (!cfg_valid(cfg, &why)) return -1;
    return sizes_of(cfg).P;
}

mlb_status mlb_workspace_bytes(const mlb_config* cfg, size_t* bytes) {
    std::string why;
    if (!bytes) return fail(MLB_E_INVALID_ARG, "bytes is null");
    if (!cfg_valid(cfg, &why)) return fail(MLB_E_INVALID_ARG, "%s", why.c_str());
    if (!cfg_supported(cfg, &why)) return fail(MLB_E_UNSUPPORTED, "%s", why.c_str());
    mlb_model tmp{};
    tmp.cfg = *cfg;
    tmp.s = sizes_of(cfg);
    *bytes = carve(&tmp, nullptr);
    return MLB_OK;
}

mlb_status mlb_init(const mlb_config* cfg, uint64_t seed, const float* init, void* arena, size_t arena_bytes,
                    void* stream, mlb_model** out) {
    std::string why;
    if (!out || !arena) return fail(MLB_E_INVALID_ARG, "null argument");
    *out = nullptr;
    if (!cfg_valid(cfg, &why)) return fail(MLB_E_INVALID_ARG, "%s", why.c_str());
    if (!cfg_supported(cfg, &why)) return fail(MLB_E_UNSUPPORTED, "%s", why.c_str());
    if ((uintptr_t)arena % ALIGN) return fail(MLB_E_INVALID_ARG, "arena not 256-byte aligned");
    int dev = 0;
    HIPCHK(hipGetDevice(&dev));
    hipDeviceProp_t prop;
    HIPCHK(hipGetDeviceProperties(&prop, dev));
    if (std::strncmp(prop.gcnArchName, "gfx950", 6) != 0)
        return fail(MLB_E_UNSUPPORTED, "device %s is not gfx950: the profile is certified on gfx950 only",
                    prop.gcnArchName);
    mlb_model* M = new mlb_model();
    M->cfg = *cfg;
    M->s = sizes_of(cfg);
    M->stream = static_cast<hipStream_t>(stream);
    M->device = dev;
    const size_t need = carve(M, nullptr);
    if (arena_bytes < need) {
        delete M;
        return fail(MLB_E_ARENA_TOO_SMALL, "arena holds %zu bytes, %zu needed", arena_bytes, need);
    }
    carve(M, static_cast<char*>(arena));
    offsets(M);
    M->attn_scale = (float)(1.0 / std::sqrt((double)M->s.hd));
    M->invN = 1.0f / (float)M->s.N;
    if (hipHostMalloc(reinterpret_cast<void**>(&M->host_stage), 64, hipHostMallocDefault) != hipSuccess) {
        delete M;
        return fail(MLB_E_DEVICE, "pinned staging buffer");
    }
    if (make_streams(M) != MLB_OK) {
        const mlb_status rc = MLB_E_DEVICE;
        release_streams(M);
        (void)hipHostFree(M->host_stage);
        delete M;
        return rc;
    }
    std::vector<float> drawn;
    if (!init) {
        drawn = seeded_params(M, seed);
        init = drawn.data();
    }
    std::vector<float> c, sn;
    rope_table_host(M->s.T, M->s.hd, cfg->rope_theta, c, sn);
    hipStream_t st = M->stream;
    mlb_status rc = MLB_OK;
    auto step = [&](hipError_t e, const char* what) {
        if (rc == MLB_OK && e != hipSuccess) rc = fail(MLB_E_DEVICE, "%s: %s", what, hipGetErrorString(e));
    };
    step(hipMemcpyAsync(M->p, init, (size_t)M->s.P * 4, hipMemcpyHostToDevice, st), "upload params");
    step(hipMemcpyAsync(M->cosv, c.data(), c.size() * 4, hipMemcpyHostToDevice, st), "upload rope");
    step(hipMemcpyAsync(M->sinv, sn.data(), sn.size() * 4, hipMemcpyHostToDevice, st), "upload rope");
    std::vector<int64_t> offs;
    for (int64_t l = 0; l < M->s.L; ++l) {
        offs.push_back(M->o_w2[l]);
        offs.push_back(M->o_w1[l]);
    }
    step(hipMemcpyAsync(M->dw_offs, offs.data(), offs.size() * 8, hipMemcpyHostToDevice, st), "upload gain offsets");
    if (rc == MLB_OK) {
        if (mlb::fill_zero(M->G, M->s.P, st) || mlb::fill_zero(M->m, M->s.P, st) || mlb::fill_zero(M->v, M->s.P, st))
            rc = fail(MLB_E_DEVICE, "zero fill");
    }
    step(hipStreamSynchronize(st), "init sync");
    if (rc != MLB_OK) {
        release_streams(M);
        (void)hipHostFree(M->host_stage);
        delete M;
        return rc;
    }
    M->step = 0;
    M->have_fwd = false;
    M->n_accum = 0;
    *out = M;
    return MLB_OK;
}

mlb_status mlb_forward_loss(mlb_model* M, const int32_t* d_inputs, const int32_t* d_targets, float* out_loss) {
    if (!M || !d_inputs || !d_targets || !out_loss) return fail(MLB_E_INVALID_ARG, "null argument");
    HIPCHK(hipSetDevice(M->device));
    M->have_fwd = false;
    const size_t nb = (size_t)M->s.N * 4;
    HIPCHK(hipMemcpyAsync(M->ids, d_inputs, nb, hipMemcpyDeviceToDevice, M->stream));
    HIPCHK(hipMemcpyAsync(M->tg, d_targets, nb, hipMemcpyDeviceToDevice, M->stream));
    KCHK(mlb::fill_zero(reinterpret_cast<float*>(M->err), 1, M->stream));
    mlb_status rc = forward(M);
    if (rc != MLB_OK) return rc;
    HIPCHK(hipMemcpyAsync(M->host_stage, M->loss_dev, 4, hipMemcpyDeviceToHost, M->stream));
    HIPCHK(hipMemcpyAsync(M->host_stage + 1, M->err, 4, hipMemcpyDeviceToHost, M->stream));
    HIPCHK(hipStreamSynchronize(M->stream));
    stat_resolve(M);
    int err;
    std::memcpy(&err, M->host_stage + 1, 4);
    if (err) return fail(MLB_E_BAD_TOKEN, "token id outside [0, %u) in %s", M->cfg.vocab,
                         (err & 1) ? "inputs" : "targets");
    *out_loss = M->host_stage[0];
    M->have_fwd = true;
    return MLB_OK;
}

mlb_status mlb_infer(mlb_model* M, const int32_t* d_inputs, const int32_t* d_targets, float* d_logits,
                     float* out_loss) {
    if (!M || !d_inputs || (d_targets && !out_loss) || (!d_targets && out_loss))
        return fail(MLB_E_INVALID_ARG, "null argument (targets and loss go together)");
    HIPCHK(hipSetDevice(M->device));
    if (M->have_fwd) return fail(MLB_E_STATE, "a training forward is pending its backward");
    const size_t nb = (size_t)M->s.N * 4;
    HIPCHK(hipMemcpyAsync(M->ids, d_inputs, nb, hipMemcpyDeviceToDevice, M->stream));
    if (d_targets) HIPCHK(hipMemcpyAsync(M->tg, d_targets, nb, hipMemcpyDeviceToDevice, M->stream));
    KCHK(mlb::fill_zero(reinterpret_cast<float*>(M->err), 1, M->stream));
    mlb_status rc = forward(M, d_targets ? 1 : 2);
    if (rc != MLB_OK) return rc;
    if (d_logits)
        HIPCHK(hipMemcpy2DAsync(d_logits, (size_t)M->s.V * 4, M->logits, (size_t)M->s.ldV * 4, (size_t)M->s.V * 4,
                                (size_t)M->s.N, hipMemcpyDeviceToDevice, M->stream));
    HIPCHK(hipMemcpyAsync(M->host_stage, M->loss_dev, 4, hipMemcpyDeviceToHost, M->stream));
    HIPCHK(hipMemcpyAsync(M->host_stage + 1, M->err, 4, hipMemcpyDeviceToHost, M->stream));
    HIPCHK(hipStreamSynchronize(M->stream));
    stat_resolve(M);
    int err;
    std::memcpy(&err, M->host_stage + 1, 4);
    if (err) return fail(MLB_E_BAD_TOKEN, "token id outside [0, %u) in %s", M->cfg.vocab,
                         (err & 1) ? "inputs" : "targets");
    if (out_loss) *out_loss = M->host_stage[0];
    return MLB_OK;
}

mlb_status mlb_greedy_next(mlb_model* M, const int32_t* d_inputs, int position, int32_t* next_host) {
    if (!M || !d_inputs || !next_host) return fail(MLB_E_INVALID_ARG, "null argument");
    if (position < 0 || position >= (int)M->s.T) return fail(MLB_E_INVALID_ARG, "position %d outside the window", position);
    HIPCHK(hipSetDevice(M->device));
    if (M->have_fwd) return fail(MLB_E_STATE, "a training forward is pending its backward");
    HIPCHK(hipMemcpyAsync(M->ids, d_inputs, (size_t)M->s.N * 4, hipMemcpyDeviceToDevice, M->stream));
    KCHK(mlb::fill_zero(reinterpret_cast<float*>(M->err), 1, M->stream));
    mlb_status rc = forward(M, 2);
    if (rc != MLB_OK) return rc;
    // one token per sequence: rows b * T + position of the logits; the choices
    // land in the (unused) target buffer, then go to the host
    M->cur = M->stream;
    OP("argmax", 4.0 * (double)M->s.B * (double)M->s.V,
       mlb::argmax_rows(M->logits, M->s.B, M->s.T, position, M->s.ldV, M->s.V, M->tg, M->stream));
    HIPCHK(hipMemcpyAsync(M->host_stage + 1, M->err, 4, hipMemcpyDeviceToHost, M->stream));
    std::vector<int32_t> host((size_t)M->s.B);
    HIPCHK(hipMemcpyAsync(host.data(), M->tg, host.size() * 4, hipMemcpyDeviceToHost, M->stream));
    HIPCHK(hipStreamSynchronize(M->stream));
    stat_resolve(M);
    int err;
    std::memcpy(&err, M->host_stage + 1, 4);
    if (err) return fail(MLB_E_BAD_TOKEN, "token id outside [0, %u) in inputs", M->cfg.vocab);
    std::memcpy(next_host, host.data(), host.size() * 4);
    return MLB_OK;
}

mlb_status mlb_backward(mlb_model* M) {
    if (!M) return fail(MLB_E_INVALID_ARG, "null model");
    if (!M->have_fwd) return fail(MLB_E_STATE, "backward needs a successful forward of the same micro-batch");
    HIPCHK(hipSetDevice(M->device));
    mlb_status rc = backward(M);
    if (rc != MLB_OK) return rc;
    M->have_fwd = false;
    M->n_accum += 1;
    return MLB_OK;
}

mlb_status mlb_adamw_step(mlb_model* M, float lr) {
    if (!M) return fail(MLB_E_INVALID_ARG, "null model");
    if (M->n_accum < 1) return fail(MLB_E_STATE, "no gradient accumulated since the last step");
    HIPCHK(hipSetDevice(M->device));
    const uint64_t t = M->step + 1;
    const float bc1 = bias_corr(M->cfg.beta1, t), bc2 = bias_corr(M->cfg.beta2, t);
    M->cur = M->stream;
    OP("adamw", 4.0 * 8 * (double)M->s.P,
       mlb::adamw(M->p, M->G, M->m, M->v, M->s.P, lr, M->cfg.beta1, M->cfg.beta2, M->cfg.adam_eps,
                  M->cfg.weight_decay, bc1, bc2, M->stream));
    M->step = t;
    M->n_accum = 0;
    M->have_fwd = false;
    return MLB_OK;
}

namespace {
constexpr size_t HDR = 256;

void put32(uint8_t* p, uint32_t v) { std::memcpy(p, &v, 4); }   // little-endian host
void put64(uint8_t* p, uint64_t v) { std::memcpy(p, &v, 8); }

void header(const mlb_config& c, uint64_t step, uint64_t n, const uint8_t dp[32], const uint8_t dm[32],
            const uint8_t dv[32], uint8_t* h) {
    std::memset(h, 0, HDR);
    std::memcpy(h, "MLBCKPT1", 8);
    put32(h + 8, 1u);
    put32(h + 12, MLB_PROFILE_VERSION);
    const uint32_t ci[9] = {c.vocab, c.d_model, c.n_layers, c.n_heads, c.head_dim, c.ffn_hidden, c.tied, c.batch,
                            c.seq_len};
    std::memcpy(h + 16, ci, 36);
    const float cf[6] = {c.rope_theta, c.rms_eps, c.beta1, c.beta2, c.adam_eps, c.weight_decay};
    std::memcpy(h + 52, cf, 24);
    put64(h + 80, step);
    put64(h + 88, n);
    std::memcpy(h + 96, dp, 32);
    std::memcpy(h + 128, dm, 32);
    std::memcpy(h + 160, dv, 32);
    sha256_bytes(h, 192, h + 192);
}
}  // namespace

mlb_status mlb_save(const mlb_model* M, void* buf, size_t cap, size_t* len) {
    if (!M || !len) return fail(MLB_E_INVALID_ARG, "null argument");
    const size_t nb = (size_t)M->s.P * 4, total = HDR + 3 * nb;
    *len = total;
    if (!buf) return MLB_OK;
    if (M->n_accum != 0) return fail(MLB_E_STATE, "save with pending accumulated gradients");
    if (cap < total) return fail(MLB_E_IO, "buffer holds %zu bytes, %zu needed", cap, total);
    HIPCHK(hipSetDevice(M->device));
    uint8_t* b = static_cast<uint8_t*>(buf);
    HIPCHK(hipStreamSynchronize(M->stream));
    HIPCHK(hipMemcpy(b + HDR, M->p, nb, hipMemcpyDeviceToHost));
    HIPCHK(hipMemcpy(b + HDR + nb, M->m, nb, hipMemcpyDeviceToHost));
    HIPCHK(hipMemcpy(b + HDR + 2 * nb, M->v, nb, hipMemcpyDeviceToHost));
    uint8_t dp[32], dm[32], dv[32];
    sha256_bytes(b + HDR, nb, dp);
    sha256_bytes(b + HDR + nb, nb, dm);
    sha256_bytes(b + HDR + 2 * nb, nb, dv);
    header(M->cfg, M->step, (uint64_t)M->s.P, dp, dm, dv, b);
    return MLB_OK;
}

mlb_status mlb_load(mlb_model* M, const void* buf, size_t len) {
    if (!M || !buf) return fail(MLB_E_INVALID_ARG, "null argument");
    const uint8_t* b = static_cast<const uint8_t*>(buf);
    if (len < HDR) return fail(MLB_E_CORRUPT, "truncated header");
    if (std::memcmp(b, "MLBCKPT1", 8) != 0) return fail(MLB_E_PROFILE_MISMATCH, "not an MLBC checkpoint");
    uint32_t fmt, prof;
    std::memcpy(&fmt, b + 8, 4);
    std::memcpy(&prof, b + 12, 4);
    if (fmt != 1u || prof != MLB_PROFILE_VERSION)
        return fail(MLB_E_PROFILE_MISMATCH, "format %u profile %u (expected 1, %u)", fmt, prof, MLB_PROFILE_VERSION);
    uint8_t hd[32];
    sha256_bytes(b, 192, hd);
    if (std::memcmp(hd, b + 192, 32) != 0) return fail(MLB_E_CORRUPT, "header digest mismatch");
    uint8_t zeros[32] = {0};
    if (std::memcmp(b + 224, zeros, 32) != 0 || b[76] | b[77] | b[78] | b[79])
        return fail(MLB_E_CORRUPT, "header padding not zero");
    const mlb_config& c = M->cfg;
    const uint32_t ci[9] = {c.vocab, c.d_model, c.n_layers, c.n_heads, c.head_dim, c.ffn_hidden, c.tied, c.batch,
                            c.seq_len};
    const float cf[6] = {c.rope_theta, c.rms_eps, c.beta1, c.beta2, c.adam_eps, c.weight_decay};
    if (std::memcmp(b + 16, ci, 36) != 0 || std::memcmp(b + 52, cf, 24) != 0)
        return fail(MLB_E_CONFIG_MISMATCH, "checkpoint config differs from the model's");
    uint64_t step, n;
    std::memcpy(&step, b + 80, 8);
    std::memcpy(&n, b + 88, 8);
    const size_t nb = (size_t)M->s.P * 4;
    if (n != (uint64_t)M->s.P || len != HDR + 3 * nb) return fail(MLB_E_CORRUPT, "size mismatch");
    uint8_t d3[3][32];
    for (int i = 0; i < 3; ++i) {
        sha256_bytes(b + HDR + i * nb, nb, d3[i]);
        if (std::memcmp(d3[i], b + 96 + 32 * i, 32) != 0) return fail(MLB_E_CORRUPT, "array %d digest mismatch", i);
    }
    HIPCHK(hipSetDevice(M->device));
    HIPCHK(hipStreamSynchronize(M->stream));
    HIPCHK(hipMemcpy(M->p, b + HDR, nb, hipMemcpyHostToDevice));
    HIPCHK(hipMemcpy(M->m, b + HDR + nb, nb, hipMemcpyHostToDevice));
    HIPCHK(hipMemcpy(M->v, b + HDR + 2 * nb, nb, hipMemcpyHostToDevice));
    KCHK(mlb::fill_zero(M->G, M->s.P, M->stream));
    HIPCHK(hipStreamSynchronize(M->stream));
    M->step = step;
    M->n_accum = 0;
    M->have_fwd = false;
    return MLB_OK;
}

mlb_status mlb_safetensors(const mlb_config* cfg, const float* params, void* buf, size_t cap, size_t* len) {
    std::string why;
    if (!len) return fail(MLB_E_INVALID_ARG, "len is null");
    if (!cfg_valid(cfg, &why)) return fail(MLB_E_INVALID_ARG, "%s", why.c_str());
    const Sizes s = sizes_of(cfg);
    char num[96];
    std::string h = "{\"__metadata__\":{\"format\":\"pt\",\"profile\":\"MLB-P1\"";
    const std::pair<const char*, uint32_t> ints[] = {{"vocab", cfg->vocab},         {"d_model", cfg->d_model},
                                                     {"n_layers", cfg->n_layers},   {"n_heads", cfg->n_heads},
                                                     {"head_dim", cfg->head_dim},   {"ffn_hidden", cfg->ffn_hidden},
                                                     {"tied", cfg->tied}};
    for (const auto& kv : ints) {
        std::snprintf(num, sizeof num, ",\"%s\":\"%u\"", kv.first, kv.second);
        h += num;
    }
    // 9 significant digits carry a binary32 value exactly through decimal
    std::snprintf(num, sizeof num, ",\"rope_theta\":\"%.9g\",\"rms_eps\":\"%.9g\"}", (double)cfg->rope_theta,
                  (double)cfg->rms_eps);
    h += num;
    int64_t off = 0;   // byte offset in the data section; tensors in canonical order
    auto add = [&](const std::string& name, int64_t rows, int64_t cols) {
        const int64_t nb = rows * (cols ? cols : 1) * 4;
        if (cols) std::snprintf(num, sizeof num, "[%lld,%lld]", (long long)rows, (long long)cols);
        else std::snprintf(num, sizeof num, "[%lld]", (long long)rows);
        h += ",\"" + name + "\":{\"dtype\":\"F32\",\"shape\":" + num;
        std::snprintf(num, sizeof num, ",\"data_offsets\":[%lld,%lld]}", (long long)off, (long long)(off + nb));
        h += num;
        off += nb;
    };
    add("E_in", s.V, s.d);
    for (int64_t l = 0; l < s.L; ++l) {
        const std::string pre = "l" + std::to_string(l) + ".";
        add(pre + "attn_norm", s.d, 0);
        add(pre + "Wq", s.d, s.d); add(pre + "Wk", s.d, s.d); add(pre + "Wv", s.d, s.d); add(pre + "Wo", s.d, s.d);
        add(pre + "mlp_norm", s.d, 0);
        add(pre + "Wg", s.F, s.d); add(pre + "Wu", s.F, s.d); add(pre + "Wd", s.d, s.F);
    }
    if (!s.tied) add("W_out", s.V, s.d);
    h += "}";
    while (h.size() % 8) h += ' ';   // the format allows trailing spaces; keeps the data 8-byte aligned
    if (off != s.P * 4) return fail(MLB_E_INVALID_ARG, "internal: tensor table covers %lld of %lld bytes",
                                    (long long)off, (long long)(s.P * 4));
    const size_t total = 8 + h.size() + (size_t)off;
    *len = total;
    if (!buf) return MLB_OK;
    if (!params) return fail(MLB_E_INVALID_ARG, "params is null");
    if (cap < total) return fail(MLB_E_IO, "buffer holds %zu bytes, %zu needed", cap, total);
    uint8_t* b = static_cast<uint8_t*>(buf);
    put64(b, (uint64_t)h.size());
    std::memcpy(b + 8, h.data(), h.size());
    std::memcpy(b + 8 + h.size(), params, (size_t)off);
    return MLB_OK;
}

mlb_status mlb_read(const mlb_model* M, mlb_which w, void* dst, size_t bytes) {
    if (!M || !dst) return fail(MLB_E_INVALID_ARG, "null argument");
    const size_t nb = (size_t)M->s.P * 4;
    if (bytes < nb) return fail(MLB_E_IO, "buffer holds %zu bytes, %zu needed", bytes, nb);
    const float* src = w == MLB_PARAMS ? M->p : w == MLB_GRAD ? M->G : w == MLB_ADAM_M ? M->m : w == MLB_ADAM_V ? M->v
                                                                                                                 : nullptr;
    if (!src) return fail(MLB_E_INVALID_ARG, "unknown array %d", (int)w);
    HIPCHK(hipSetDevice(M->device));
    HIPCHK(hipStreamSynchronize(M->stream));
    HIPCHK(hipMemcpy(dst, src, nb, hipMemcpyDeviceToHost));
    return MLB_OK;
}

mlb_status mlb_read_stage(const mlb_model* M, int stage, int layer, void* dst, size_t bytes, size_t* count) {
    if (!M || !count) return fail(MLB_E_INVALID_ARG, "null argument");
    const Sizes& s = M->s;
    if (layer < 0 || layer >= s.L) return fail(MLB_E_INVALID_ARG, "layer %d out of range", layer);
    const float* src = nullptr;
    int64_t n = 0;
    switch (stage) {
        case 0: src = M->h[layer]; n = s.N * s.d; break;
        case 1: src = M->xn1[layer]; n = s.N * s.d; break;
        case 2: src = M->r1[layer]; n = s.N; break;
        case 3: src = M->qkv[layer]; n = s.N * 3 * s.d; break;
        case 4: src = M->P[layer]; n = s.B * s.H * s.T * s.T; break;
        case 5: src = M->O[layer]; n = s.N * s.d; break;
        case 6: src = M->hmid[layer]; n = s.N * s.d; break;
        case 7: src = M->xn2[layer]; n = s.N * s.d; break;
        case 8: src = M->r2[layer]; n = s.N; break;
        case 9: src = M->gu[layer]; n = s.N * 2 * s.F; break;
        case 10: src = M->a[layer]; n = s.N * s.F; break;
        case 11: src = M->h[s.L]; n = s.N * s.d; break;
        case 12: src = M->logits; n = s.N * s.V; break;   // rows compacted from the padded stride
        case 13: src = M->loss_rows; n = s.N; break;
        case 14: src = M->cosv; n = s.T * (s.hd / 2); break;   // rotary tables [T, hd/2]
        case 15: src = M->sinv; n = s.T * (s.hd / 2); break;
        default: return fail(MLB_E_INVALID_ARG, "unknown stage %d", stage);
    }
    *count = (size_t)n;
    if (!dst) return MLB_OK;
    if (bytes < (size_t)n * 4) return fail(MLB_E_IO, "buffer too small");
    HIPCHK(hipSetDevice(M->device));
    HIPCHK(hipStreamSynchronize(M->stream));
    if (stage == 12) {
        HIPCHK(hipMemcpy2D(dst, (size_t)s.V * 4, src, (size_t)s.ldV * 4, (size_t)s.V * 4, (size_t)s.N,
                           hipMemcpyDeviceToHost));
    } else if (stage == 4) {   // tiled on the device, dense [B*H, T, T] for the caller
        std::vector<float> tmp((size_t)n);
        HIPCHK(hipMemcpy(tmp.data(), src, (size_t)n * 4, hipMemcpyDeviceToHost));
        float* o = static_cast<float*>(dst);
        for (int64_t z = 0; z < s.B * s.H; ++z)
            for (int64_t i = 0; i < s.T; ++i)
                for (int64_t j = 0; j < s.T; ++j)   // +0 above the diagonal (never part of P)
                    o[(z * s.T + i) * s.T + j] =
                        j <= i ? tmp[(size_t)(z * s.T * s.T + mlb::blk_index(s.T, i, j))] : 0.0f;
    } else {
        HIPCHK(hipMemcpy(dst, src, (size_t)n * 4, hipMemcpyDeviceToHost));
    }
    return MLB_OK;
}

mlb_status mlb_stage_card(const mlb_model* M, int stage, int layer, mlb_card* out) {
    static const char* const names[14] = {"h_in", "xn1", "r1", "qkv", "P", "O", "h_mid",
                                          "xn2", "r2", "gu", "a", "h_L", "dlogits", "loss_rows"};
    if (!M || !out) return fail(MLB_E_INVALID_ARG, "null argument");
    if (stage < 0 || stage > 13) return fail(MLB_E_INVALID_ARG, "unknown stage %d", stage);
    size_t n = 0;
    mlb_status rc = mlb_read_stage(M, stage, layer, nullptr, 0, &n);
    if (rc != MLB_OK) return rc;
    std::vector<float> host(n);
    rc = mlb_read_stage(M, stage, layer, host.data(), n * 4, &n);
    if (rc != MLB_OK) return rc;
    std::memset(out, 0, sizeof *out);
    if (stage <= 10) std::snprintf(out->tag, sizeof out->tag, "L%d.%s", layer, names[stage]);
    else std::snprintf(out->tag, sizeof out->tag, "%s", names[stage]);
    std::snprintf(out->dtype, sizeof out->dtype, "f32");
    out->count = n;
    sha256_bytes(host.data(), n * 4, out->sha256);
    return MLB_OK;
}

mlb_status mlb_state_card(const mlb_model* M, mlb_which which, mlb_card* out) {
    static const char* const names[4] = {"params", "grad", "adam_m", "adam_v"};
    if (!M || !out) return fail(MLB_E_INVALID_ARG, "null argument");
    if (which < MLB_PARAMS || which > MLB_ADAM_V) return fail(MLB_E_INVALID_ARG, "unknown state array");
    std::vector<float> host((size_t)M->s.P);
    const mlb_status rc = mlb_read(M, which, host.data(), host.size() * 4);
    if (rc != MLB_OK) return rc;
    std::memset(out, 0, sizeof *out);
    std::snprintf(out->tag, sizeof out->tag, "%s", names[which]);
    std::snprintf(out->dtype, sizeof out->dtype, "f32");
    out->count = (uint64_t)M->s.P;
    sha256_bytes(host.data(), host.size() * 4, out->sha256);
    return MLB_OK;
}

uint64_t mlb_step(const mlb_model* M) { return M ? M->step : 0; }

mlb_status mlb_destroy(mlb_model* M) {
    if (!M) return MLB_OK;
    (void)hipSetDevice(M->device);
    (void)hipStreamSynchronize(M->stream);
    release_streams(M);
    stat_resolve(M);
    for (hipEvent_t e : M->free_events) (void)hipEventDestroy(e);
    (void)hipHostFree(M->host_stage);
    delete M;
    return MLB_OK;
}

mlb_status mlb_set_overlap(mlb_model* M, int on) {
    if (!M) return fail(MLB_E_INVALID_ARG, "null model");
    if (M->have_fwd) return fail(MLB_E_STATE, "a forward is pending its backward");
    HIPCHK(hipSetDevice(M->device));
    HIPCHK(hipStreamSynchronize(M->stream));
    M->overlap = on != 0;
    return MLB_OK;
}

mlb_status mlb_stats_enable(mlb_model* M, int on) {
    if (!M) return fail(MLB_E_INVALID_ARG, "null model");
    HIPCHK(hipSetDevice(M->device));
    HIPCHK(hipStreamSynchronize(M->stream));
    stat_resolve(M);
    M->agg.clear();
    M->stats_on = on != 0;
    return MLB_OK;
}

mlb_status mlb_stats_sites(mlb_model* M, const char* sites) {
    if (!M) return fail(MLB_E_INVALID_ARG, "null model");
    M->stats_sites.clear();
    if (!sites) return MLB_OK;
    std::string cur;
    for (const char* c = sites;; ++c) {
        if (*c == ',' || *c == '\0') {
            if (!cur.empty()) M->stats_sites.push_back(cur);
            cur.clear();
            if (*c == '\0') break;
        } else {
            cur += *c;
        }
    }
    return MLB_OK;
}

mlb_status mlb_stats_read(mlb_model* M, mlb_stat* out, int cap, int* n) {
    if (!M || !n) return fail(MLB_E_INVALID_ARG, "null argument");
    HIPCHK(hipSetDevice(M->device));
    HIPCHK(hipStreamSynchronize(M->stream));
    stat_resolve(M);
    *n = (int)M->agg.size();
    int i = 0;
    for (const auto& kv : M->agg) {
        if (!out || i >= cap) break;
        mlb_stat& o = out[i++];
        std::memset(&o, 0, sizeof o);
        std::snprintf(o.site, sizeof o.site, "%s", kv.second.site.c_str());
        std::snprintf(o.kernel, sizeof o.kernel, "%s", kv.second.kernel.c_str());
        o.launches = kv.second.launches;
        o.ms = kv.second.ms;
        o.flops = kv.second.flops;
        o.bytes = kv.second.bytes;
    }
    return MLB_OK;
}

const char* mlb_status_name(mlb_status s) {
    switch (s) {
        case MLB_OK: return "MLB_OK";
        case MLB_E_INVALID_ARG: return "MLB_E_INVALID_ARG";
        case MLB_E_UNSUPPORTED: return "MLB_E_UNSUPPORTED";
        case MLB_E_DEVICE: return "MLB_E_DEVICE";
        case MLB_E_ARENA_TOO_SMALL: return "MLB_E_ARENA_TOO_SMALL";
        case MLB_E_BAD_TOKEN: return "MLB_E_BAD_TOKEN";
        case MLB_E_STATE: return "MLB_E_STATE";
        case MLB_E_CORRUPT: return "MLB_E_CORRUPT";
        case MLB_E_PROFILE_MISMATCH: return "MLB_E_PROFILE_MISMATCH";
        case MLB_E_CONFIG_MISMATCH: return "MLB_E_CONFIG_MISMATCH";
        case MLB_E_IO: return "MLB_E_IO";
        default: return "MLB_E_UNKNOWN";
    }
}

const char* mlb_last_error_message(void) { return g_msg; }
uint32_t mlb_profile_version(void) { return MLB_PROFILE_VERSION; }

// ------------------------------------------------------------- primitives
mlb_status mlb_prim_gemm(int64_t M, int64_t N, int64_t K, int64_t kseg, const float* A, int64_t lda, int a_kc,
                         const float* B, int64_t ldb, int b_kc, float* C, int64_t ldc, int krange, int outmask,
                         int mode, float scale, int64_t batch, int64_t heads, int64_t sAb, int64_t sAh, int64_t sBb,
                         int64_t sBh, int64_t sCb, int64_t sCh, int tile, int split, int simple, void* ws,
                         size_t ws_bytes, void* stream) {
    if (mode < 0 || mode > 2) return fail(MLB_E_INVALID_ARG, "mode %d", mode);
    mlb::GemmDesc g;
    g.M = M; g.N = N; g.K = K; g.kseg = kseg > 0 ? kseg : K;
    g.A = A; g.lda = lda; g.a_kc = a_kc != 0; g.B = B; g.ldb = ldb; g.b_kc = b_kc != 0; g.C = C; g.ldc = ldc;
    g.krange = krange; g.outmask = outmask; g.mode = mode; g.scale = scale;
    g.batch = batch; g.H = heads; g.sAb = sAb; g.sAh = sAh; g.sBb = sBb; g.sBh = sBh; g.sCb = sCb; g.sCh = sCh;
    if (tile < -1 || tile > 2) return fail(MLB_E_INVALID_ARG, "tile %d", tile);
    mlb::GemmPlan p;
    p.tile = tile; p.split = split; p.simple = simple;
    p.scratch = static_cast<float*>(ws);
    p.scratch_floats = (int64_t)(ws_bytes / 4);
    if (split == 1 && mlb::gemm_split_scratch(g, p) > p.scratch_floats)
        return fail(MLB_E_ARENA_TOO_SMALL, "split needs %ld floats", (long)mlb::gemm_split_scratch(g, p));
    const int r = mlb::gemm(g, p, static_cast<hipStream_t>(stream));
    if (r == -1) return fail(MLB_E_INVALID_ARG, "invalid contraction description");
    if (r != 0) return fail(MLB_E_DEVICE, "contraction launch failed (%d)", r);
    return MLB_OK;
}

mlb_status mlb_prim_gemm_pair(int64_t M0, int64_t N0, int64_t M1, int64_t N1, int64_t K, const float* A0,
                              int64_t lda0, const float* B0, int64_t ldb0, float* C0, int64_t ldc0, const float* A1,
                              int64_t lda1, const float* B1, int64_t ldb1, float* C1, int64_t ldc1, int a_kc, int b_kc,
                              int mode, void* ws, size_t ws_bytes, void* stream) {
    if (mode < 0 || mode > 1) return fail(MLB_E_INVALID_ARG, "mode %d", mode);
    mlb::GemmDesc g[2];
    const int64_t Ms[2] = {M0, M1}, Ns[2] = {N0, N1}, lda[2] = {lda0, lda1}, ldb[2] = {ldb0, ldb1},
                  ldc[2] = {ldc0, ldc1};
    const float* As[2] = {A0, A1};
    const float* Bs[2] = {B0, B1};
    float* Cs[2] = {C0, C1};
    for (int i = 0; i < 2; ++i) {
        g[i].M = Ms[i]; g[i].N = Ns[i]; g[i].K = K; g[i].kseg = K;
        g[i].A = As[i]; g[i].lda = lda[i]; g[i].a_kc = a_kc != 0;
        g[i].B = Bs[i]; g[i].ldb = ldb[i]; g[i].b_kc = b_kc != 0;
        g[i].C = Cs[i]; g[i].ldc = ldc[i]; g[i].mode = mode;
    }
    mlb::GemmPlan p;
    p.scratch = static_cast<float*>(ws);
    p.scratch_floats = (int64_t)(ws_bytes / 4);
    const int r = mlb::gemm_pair(g[0], g[1], p, static_cast<hipStream_t>(stream));
    if (r == -1) return fail(MLB_E_INVALID_ARG, "invalid contraction description");
    if (r != 0) return fail(MLB_E_DEVICE, "contraction pair launch failed (%d)", r);
    return MLB_OK;
}

mlb_status mlb_prim_rmsnorm_fwd(const float* x, const float* w, int64_t rows, int64_t d, float eps, float* y, float* r,
                                void* stream) {
    if (!x || !w || !y || !r) return fail(MLB_E_INVALID_ARG, "null argument");
    return mlb::rmsnorm_fwd(x, w, rows, d, eps, y, r, static_cast<hipStream_t>(stream)) == 0
               ? MLB_OK
               : fail(MLB_E_INVALID_ARG, "rmsnorm_fwd");
}

mlb_status mlb_prim_rmsnorm_bwd(const float* dy, const float* x, const float* w, const float* r, int64_t rows,
                                int64_t d, float* dx, float* dw, void* ws, size_t ws_bytes, void* stream) {
    if (!dy || !x || !w || !r || !dx || !dw) return fail(MLB_E_INVALID_ARG, "null argument");
    const size_t need = (size_t)((rows + KCH - 1) / KCH) * (size_t)d * 4;
    if (ws_bytes < need || (!ws && need)) return fail(MLB_E_ARENA_TOO_SMALL, "rmsnorm_bwd needs %zu bytes", need);
    hipStream_t st = static_cast<hipStream_t>(stream);
    if (mlb::rmsnorm_bwd_dx(dy, x, w, r, rows, d, nullptr, dx, st) ||
        mlb::rmsnorm_bwd_dw(dy, x, r, rows, d, static_cast<float*>(ws), dw, 0, st))
        return fail(MLB_E_INVALID_ARG, "rmsnorm_bwd");
    return MLB_OK;
}

mlb_status mlb_prim_rope(float* x, int64_t B, int64_t T, int64_t H, int64_t hd, int64_t ld, float theta, int backward,
                         void* stream) {
    if (!x || hd % 2 || T <= 0) return fail(MLB_E_INVALID_ARG, "rope arguments");
    std::vector<float> c, sn;
    rope_table_host(T, hd, theta, c, sn);
    float* tab = nullptr;
    HIPCHK(hipMalloc(reinterpret_cast<void**>(&tab), c.size() * 8));
    hipStream_t st = static_cast<hipStream_t>(stream);
    HIPCHK(hipMemcpyAsync(tab, c.data(), c.size() * 4, hipMemcpyHostToDevice, st));
    HIPCHK(hipMemcpyAsync(tab + c.size(), sn.data(), c.size() * 4, hipMemcpyHostToDevice, st));
    const int r = mlb::rope(x, B, T, H, hd, ld, tab, tab + c.size(), backward, st);
    HIPCHK(hipStreamSynchronize(st));
    HIPCHK(hipFree(tab));
    return r == 0 ? MLB_OK : fail(MLB_E_INVALID_ARG, "rope");
}

mlb_status mlb_prim_attention_fwd(int64_t B, int64_t H, int64_t T, int64_t hd, const float* q, const float* k,
                                  const float* v, int64_t ld, float* P, float* O, int64_t ldo, int p_tiled, void* stream) {
    if (!q || !k || !v || !P || !O || B <= 0 || H <= 0 || T <= 0 || hd <= 0) return fail(MLB_E_INVALID_ARG, "attention");
    if (p_tiled && (T % 32 || hd > 64)) return fail(MLB_E_UNSUPPORTED, "tiled P needs T % 32 == 0 and hd <= 64");
    hipStream_t st = static_cast<hipStream_t>(stream);
    mlb::GemmPlan plan;
    const float scale = (float)(1.0 / std::sqrt((double)hd));
    const bool rows = p_tiled && mlb::attn_rows_fits(T, hd, B * H, H, q, ld, T * ld, hd, k, ld, T * ld, hd, P, T,
                                                     H * T * T, T * T);
    if (rows) {
        if (mlb::attn_rows(T, hd, B * H, H, q, ld, T * ld, hd, k, ld, T * ld, hd, P, T, H * T * T, T * T, scale,
                           nullptr, nullptr, nullptr, 0, 0, 0, nullptr, 0, 0, 0, st))
            return fail(MLB_E_DEVICE, "scores");
    } else if (hd <= 64) {
        if (mlb::tri_nt(T, hd, B * H, H, q, ld, T * ld, hd, k, ld, T * ld, hd, P, T, H * T * T, T * T, 1, scale,
                        p_tiled, nullptr, nullptr, 0.0f, st))
            return fail(MLB_E_DEVICE, "scores");
    } else {
        mlb::GemmDesc sg;
        sg.batch = B * H; sg.H = H;
        sg.M = T; sg.N = T; sg.K = hd; sg.kseg = hd;
        sg.A = q; sg.lda = ld; sg.a_kc = true; sg.sAb = T * ld; sg.sAh = hd;
        sg.B = k; sg.ldb = ld; sg.b_kc = true; sg.sBb = T * ld; sg.sBh = hd;
        sg.C = P; sg.ldc = T; sg.sCb = H * T * T; sg.sCh = T * T;
        sg.outmask = 1; sg.mode = 2; sg.scale = scale;
        if (mlb::gemm(sg, plan, st)) return fail(MLB_E_DEVICE, "scores");
    }
    if (mlb::softmax_causal(P, B * H, T, p_tiled, st)) return fail(MLB_E_DEVICE, "softmax");
    mlb::GemmDesc pv;
    pv.batch = B * H; pv.H = H;
    pv.M = T; pv.N = hd; pv.K = T; pv.kseg = T; pv.krange = 1; pv.a_blk = p_tiled != 0;
    pv.A = P; pv.lda = T; pv.a_kc = true; pv.sAb = H * T * T; pv.sAh = T * T;
    pv.B = v; pv.ldb = ld; pv.b_kc = false; pv.sBb = T * ld; pv.sBh = hd;
    pv.C = O; pv.ldc = ldo; pv.sCb = T * ldo; pv.sCh = hd;
    if (mlb::gemm(pv, plan, st)) return fail(MLB_E_DEVICE, "PV");
    return MLB_OK;
}

mlb_status mlb_prim_attention_bwd(int64_t B, int64_t H, int64_t T, int64_t hd, const float* q, const float* k,
                                  const float* v, int64_t ld, const float* P, const float* O, const float* dO,
                                  int64_t ldo, float* dq, float* dk, float* dv, int p_tiled, void* ws, size_t ws_bytes,
                                  void* stream) {
    if (!q || !k || !v || !P || !O || !dO || !dq || !dk || !dv || B <= 0 || H <= 0 || T <= 0 || hd <= 0)
        return fail(MLB_E_INVALID_ARG, "attention_bwd");
    if (p_tiled && (T % 32 || hd > 64)) return fail(MLB_E_UNSUPPORTED, "tiled P needs T % 32 == 0 and hd <= 64");
    const size_t need = (size_t)(B * H * T * T + B * H * T) * 4;
    if (!ws || ws_bytes < need) return fail(MLB_E_ARENA_TOO_SMALL, "attention_bwd needs %zu bytes", need);
    float* dP = static_cast<float*>(ws);
    float* D = dP + B * H * T * T;
    hipStream_t st = static_cast<hipStream_t>(stream);
    mlb::GemmPlan plan;
    const float scale = (float)(1.0 / std::sqrt((double)hd));
    if (mlb::attn_rowdot(dO, O, B, H, T, hd, ldo, D, st)) return fail(MLB_E_DEVICE, "rowdot");
    const bool rows = p_tiled && mlb::attn_rows_fits(T, hd, B * H, H, dO, ldo, T * ldo, hd, v, ld, T * ld, hd, dP, T,
                                                     H * T * T, T * T) &&
                      ((uintptr_t)k & 15u) == 0 && ld % 4 == 0;
    if (rows) {
        // dS and dQ in one pass
        if (mlb::attn_rows(T, hd, B * H, H, dO, ldo, T * ldo, hd, v, ld, T * ld, hd, dP, T, H * T * T, T * T, scale, P,
                           D, k, ld, T * ld, hd, dq, ld, T * ld, hd, st))
            return fail(MLB_E_DEVICE, "dS");
    } else if (hd <= 64) {
        // dS directly: the softmax backward runs in the epilogue
        if (mlb::tri_nt(T, hd, B * H, H, dO, ldo, T * ldo, hd, v, ld, T * ld, hd, dP, T, H * T * T, T * T, 0, 1.0f,
                        p_tiled, P, D, scale, st))
            return fail(MLB_E_DEVICE, "dS");
    } else {
        mlb::GemmDesc g;
        g.batch = B * H; g.H = H;
        g.M = T; g.N = T; g.K = hd; g.kseg = hd; g.outmask = 1;
        g.A = dO; g.lda = ldo; g.a_kc = true; g.sAb = T * ldo; g.sAh = hd;
        g.B = v; g.ldb = ld; g.b_kc = true; g.sBb = T * ld; g.sBh = hd;
        g.C = dP; g.ldc = T; g.sCb = H * T * T; g.sCh = T * T;
        if (mlb::gemm(g, plan, st)) return fail(MLB_E_DEVICE, "dP");
    }
    mlb::GemmDesc gv;
    gv.batch = B * H; gv.H = H;
    gv.M = T; gv.N = hd; gv.K = T; gv.kseg = T; gv.krange = 2; gv.a_blk = p_tiled != 0;
    gv.A = P; gv.lda = T; gv.a_kc = false; gv.sAb = H * T * T; gv.sAh = T * T;
    gv.B = dO; gv.ldb = ldo; gv.b_kc = false; gv.sBb = T * ldo; gv.sBh = hd;
    gv.C = dv; gv.ldc = ld; gv.sCb = T * ld; gv.sCh = hd;
    if (mlb::gemm(gv, plan, st)) return fail(MLB_E_DEVICE, "dv");
    if (hd > 64 && mlb::softmax_bwd(P, dP, D, B * H, T, scale, p_tiled, st)) return fail(MLB_E_DEVICE, "softmax_bwd");
    mlb::GemmDesc gq;
    gq.batch = B * H; gq.H = H;
    gq.M = T; gq.N = hd; gq.K = T; gq.kseg = T; gq.krange = 1; gq.a_blk = p_tiled != 0;
    gq.A = dP; gq.lda = T; gq.a_kc = true; gq.sAb = H * T * T; gq.sAh = T * T;
    gq.B = k; gq.ldb = ld; gq.b_kc = false; gq.sBb = T * ld; gq.sBh = hd;
    gq.C = dq; gq.ldc = ld; gq.sCb = T * ld; gq.sCh = hd;
    if (!rows && mlb::gemm(gq, plan, st)) return fail(MLB_E_DEVICE, "dq");
    mlb::GemmDesc gk;
    gk.batch = B * H; gk.H = H;
    gk.M = T; gk.N = hd; gk.K = T; gk.kseg = T; gk.krange = 2; gk.a_blk = p_tiled != 0;
    gk.A = dP; gk.lda = T; gk.a_kc = false; gk.sAb = H * T * T; gk.sAh = T * T;
    gk.B = q; gk.ldb = ld; gk.b_kc = false; gk.sBb = T * ld; gk.sBh = hd;
    gk.C = dk; gk.ldc = ld; gk.sCb = T * ld; gk.sCh = hd;
    if (mlb::gemm(gk, plan, st)) return fail(MLB_E_DEVICE, "dk");
    return MLB_OK;
}

mlb_status mlb_prim_swiglu_fwd(const float* gu, int64_t rows, int64_t F, float* a, void* stream) {
    if (!gu || !a) return fail(MLB_E_INVALID_ARG, "null argument");
    return mlb::swiglu_fwd(gu, rows, F, a, static_cast<hipStream_t>(stream)) == 0 ? MLB_OK
                                                                                   : fail(MLB_E_DEVICE, "swiglu_fwd");
}

mlb_status mlb_prim_swiglu_bwd(const float* dA, const float* gu, int64_t rows, int64_t F, float* dgu, void* stream) {
    if (!dA || !gu || !dgu) return fail(MLB_E_INVALID_ARG, "null argument");
    return mlb::swiglu_bwd(dA, gu, rows, F, dgu, static_cast<hipStream_t>(stream)) == 0
               ? MLB_OK
               : fail(MLB_E_DEVICE, "swiglu_bwd");
}

mlb_status mlb_prim_cross_entropy(const float* logits, const int32_t* targets, int64_t N, int64_t V, float* loss_rows,
                                  float* dl, float* loss_dev, void* stream) {
    if (!logits || !targets || !loss_rows || !dl || !loss_dev) return fail(MLB_E_INVALID_ARG, "null argument");
    hipStream_t st = static_cast<hipStream_t>(stream);
    int* err = nullptr;
    HIPCHK(hipMalloc(reinterpret_cast<void**>(&err), 4));
    HIPCHK(hipMemsetAsync(err, 0, 4, st));
    const int r = mlb::cross_entropy(logits, targets, N, V, V, loss_rows, dl, err, st);
    const int r2 = r == 0 ? mlb::sum64_scaled(loss_rows, N, 1.0f / (float)N, loss_dev, st) : r;
    int herr = 0;
    HIPCHK(hipMemcpyAsync(&herr, err, 4, hipMemcpyDeviceToHost, st));
    HIPCHK(hipStreamSynchronize(st));
    HIPCHK(hipFree(err));
    if (r || r2) return fail(MLB_E_INVALID_ARG, "cross_entropy");
    if (herr) return fail(MLB_E_BAD_TOKEN, "target outside [0, %ld)", (long)V);
    return MLB_OK;
}

mlb_status mlb_prim_embed_scatter(const int32_t* ids, const float* dh, int64_t N, int64_t d, int64_t V, float* dE,
                                  void* ws, size_t ws_bytes, void* stream) {
    if (!ids || !dh || !dE) return fail(MLB_E_INVALID_ARG, "null argument");
    if (N > MAX_TOKENS) return fail(MLB_E_UNSUPPORTED, "%ld positions: at most 65,536", (long)N);
    const size_t need = 8 * (size_t)std::max<int64_t>(2 * 8192, mlb::embed_key_slots(N));
    if (!ws || ws_bytes < need) return fail(MLB_E_ARENA_TOO_SMALL, "scatter of %ld positions needs %zu bytes", (long)N, need);
    const int r = mlb::embed_scatter(ids, dh, N, d, V, dE, dE, 0, static_cast<uint64_t*>(ws),
                                     static_cast<hipStream_t>(stream));
    return r == 0 ? MLB_OK : fail(MLB_E_INVALID_ARG, "embed_scatter (%d)", r);
}

// Allocation-free scatter: the sort keys live in a file-scope device array
// (one copy per GPU, held until the process ends). Host code must not pass the
// array's name to a kernel (on the host it is only a stand-in symbol): its
// device address is looked up once per device with hipGetSymbolAddress and
// that address is what the kernels receive.
constexpr int64_t SCATTER_SCRATCH_KEYS = 8192;   // 64 KiB of sort keys
static __device__ __align__(256) uint64_t scratch[SCATTER_SCRATCH_KEYS];

namespace {
constexpr int MAX_DEVICES = 64;
std::once_flag g_scratch_once[MAX_DEVICES];
uint64_t* g_scratch_ptr[MAX_DEVICES];
hipError_t g_scratch_err[MAX_DEVICES];
}  // namespace

mlb_status mlb_prim_embed_scatter_noalloc(const int32_t* ids, const float* dh, int64_t N, int64_t d, int64_t V,
                                          float* dE, void* stream) {
    if (!ids || !dh || !dE) return fail(MLB_E_INVALID_ARG, "null argument");
    if (N < 0 || d <= 0 || V <= 0) return fail(MLB_E_INVALID_ARG, "sizes N %ld, d %ld, V %ld", (long)N, (long)d, (long)V);
    if (N > SCATTER_SCRATCH_KEYS)
        return fail(MLB_E_UNSUPPORTED, "%ld positions: the static scratch holds the keys of at most %ld", (long)N,
                    (long)SCATTER_SCRATCH_KEYS);
    int dev = 0;
    HIPCHK(hipGetDevice(&dev));
    if (dev < 0 || dev >= MAX_DEVICES) return fail(MLB_E_DEVICE, "device %d beyond the scratch table", dev);
    std::call_once(g_scratch_once[dev], [dev] {
        void* ptr = nullptr;
        g_scratch_err[dev] = hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch));
        g_scratch_ptr[dev] = static_cast<uint64_t*>(ptr);
    });
    if (g_scratch_err[dev] != hipSuccess || !g_scratch_ptr[dev])
        return fail(MLB_E_DEVICE, "scratch address on device %d: %s", dev, hipGetErrorString(g_scratch_err[dev]));
    const int r = mlb::embed_scatter(ids, dh, N, d, V, dE, dE, 0, g_scratch_ptr[dev], static_cast<hipStream_t>(stream));
    return r == 0 ? MLB_OK : fail(MLB_E_DEVICE, "embed_scatter (%d)", r);
}

mlb_status mlb_prim_adamw(float* p, float* g, float* m, float* v, int64_t n, float lr, float beta1, float beta2,
                          float eps, float wd, int64_t t, void* stream) {
    if (!p || !g || !m || !v || t < 1) return fail(MLB_E_INVALID_ARG, "adamw arguments");
    const int r = mlb::adamw(p, g, m, v, n, lr, beta1, beta2, eps, wd, bias_corr(beta1, (uint64_t)t),
                             bias_corr(beta2, (uint64_t)t), static_cast<hipStream_t>(stream));
    return r == 0 ? MLB_OK : fail(MLB_E_DEVICE, "adamw");
}

mlb_status mlb_prim_unary(const float* x, float* y, int64_t n, int which, void* stream) {
    if (!x || !y) return fail(MLB_E_INVALID_ARG, "null argument");
    return mlb::exp_array(x, y, n, which, static_cast<hipStream_t>(stream)) == 0 ? MLB_OK
                                                                                  : fail(MLB_E_INVALID_ARG, "unary");
}

mlb_status mlb_diag_mfma(int variant, const float* A, const float* B, const float* C, float* D, int64_t nwaves,
                         void* stream) {
    if (!A || !B || !C || !D) return fail(MLB_E_INVALID_ARG, "null argument");
    return mlb::mfma_probe(variant, A, B, C, D, nwaves, static_cast<hipStream_t>(stream)) == 0
               ? MLB_OK
               : fail(MLB_E_INVALID_ARG, "variant %d", variant);
}

}  // extern "C"
