/*
 * latentmoe_oracle.c -- plain fp64 CPU reference of the LatentMoE layer forward.
 *
 * TEST INFRASTRUCTURE ONLY.  Only the test suite, the smoke check and the
 * benchmark's CPU-baseline leg may load or call this file.  It shares no code,
 * header, table or helper with the HIP library, and the HIP library never
 * calls it.
 *
 * What it computes (one token at a time, in the order the pages give):
 *   1. z = W_down x: the token of width d is projected to the latent width l
 *      (qingkeai.online LatentMoE article, section "LatentMoE 具体怎么做",
 *      first bullet; zhichai.net "LatentMoE: How MoE Made a Key Paradigm Leap
 *      in 2026", section 2, step 1; 10100.com article section 2.2, Figure 3b).
 *   2. Router logits from x at the full width d: the gate is one of the parts
 *      that stay at d (qingkeai.online article, closing paragraph of
 *      "LatentMoE 具体怎么做"; zhichai.net section 2, last paragraph).  Other
 *      sentences of the same pages say routing happens in l; the full-d
 *      reading is the one taken here.
 *   3. Softmax over all N logits, keep the K largest (ties: lower expert index
 *      first), renormalise the kept probabilities to sum 1.  The pages name
 *      top-K counts (512/top-22, 896/top-16: zhichai.net section 4) but not
 *      the gate function; this is the reading taken.
 *   4. Each selected expert runs in the latent space: h = W1[e] z,
 *      a = max(h, 0)^2, y = W2[e] a; its weights are l x m instead of d x m
 *      (qingkeai.online article, "LatentMoE 具体怎么做", second bullet and the
 *      paragraph after it).  The squared-ReLU activation is a reading: the
 *      pages do not name one.
 *   5. s = sum_k g_k y_k in rank order, aggregated in l before projecting back
 *      (10100.com article section 2.2: aggregate, then up-project).
 *   6. out = x + W_up s (third bullet of the same qingkeai.online section).
 *      The residual add is a reading: the pages do not state one.
 *   7. Optional shared expert at the full width d (m_shared > 0): a dense
 *      FFN on x beside the routed path, its output added to the layer's:
 *      out += Ws2 max(Ws1 x, 0)^2.  The shared expert stays at d
 *      (qingkeai.online article, closing paragraph of "LatentMoE 具体怎么做";
 *      zhichai.net section 2, last paragraph) and its output is summed with
 *      the routed one (10100.com article section 3.3, the shared-expert
 *      stream).  Its width m_shared and its activation (the routed experts'
 *      squared ReLU) are readings: the pages give neither.
 *   8. Optional zero-computation experts (10100.com article section 3.2,
 *      after MoE++): n_zero + n_copy + n_const extra expert ids N, N+1, ...
 *      (zero experts first, then copy, then constant) that the router scores
 *      like the others (W_router and bias have a row for each) and that take
 *      part in the softmax, the top-K and the renormalisation like the
 *      others.  Selected, they add g * y to s with y = 0 (zero expert: the
 *      token's input to this expert is dropped), y = z (copy expert: the
 *      identity on the expert's input) or y = c_q (constant expert: the
 *      input replaced by its own vector c_q of width l).  That they live
 *      where the routed experts live (in l, their input being z) is the
 *      reading taken; the pages describe them for a plain MoE.
 * Standard mode (no projections, l == d): z = x and out = x + s, the plain
 * MoE of 10100.com Figure 3a (plus the shared expert when present).
 *
 * Storage (row-major; the reduction index is the fastest one):
 *   x [T,d]  W_down [l,d]  W_router [Nr,d]  W1 [N,m,l]  W2 [N,l,m]  W_up [d,l]
 *   Ws1 [m_shared,d]  Ws2 [d,m_shared]  bias [Nr] float32 or NULL
 *   zc [n_const,l] (constant experts' vectors, the layer's element type)
 * with Nr = N + n_zero + n_copy + n_const routed ids.
 * Element type of x and the weights: float32 (dtype 0) or bfloat16 bit
 * patterns (dtype 1).  Each element is widened to double at use; every sum is
 * accumulated in double in index order.
 * Optional FP8 expert weights (expert_format = 1): W1 and W2 hold OCP FP8
 * E4M3 codes (one byte each: sign, 4 exponent bits with bias 7, 3 mantissa
 * bits; exponent 0 is subnormal, 0x7F / 0xFF are NaN, no infinities), with
 * one float32 scale per output row: W1[e][j][i] = e4m3(code) * s1[e*m + j],
 * W2[e][i][j] = e4m3(code) * s2[e*l + i].  The pages name low-precision
 * expert weights (NVFP4, MXFP4) without a format; this block-free per-row
 * FP8 format is a reading.
 * Optional MXFP4 expert weights (expert_format = 2; the OCP microscaling
 * format the pages name): W1 and W2 hold E2M1 codes (4 bits: sign, 2
 * exponent bits with bias 1, 1 mantissa bit; exponent 0 is subnormal; no
 * infinities or NaN), two per byte with the even element in the low nibble,
 * so W1 is [N, m, l/2] bytes and W2 [N, l, m/2]; every 32 consecutive
 * elements along the reduction index share one E8M0 scale byte (2^(b-127),
 * 0xFF is NaN): s1 [N, m, l/32] and s2 [N, l, m/32] bytes.  Element i of the
 * flattened matrix is e2m1(nibble i) * e8m0(scale byte i / 32).  The nibble
 * order and the block's direction are readings.
 *
 * Parity pins: see tests/test_oracle_pins.py.  Every output here is pinned by
 * at least one check that does not re-run this code's formulas: brute-force
 * subset enumeration for the routing, numpy float64 matmuls for the dense
 * reductions, identity and zero-weight special cases, and exact scalings.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

typedef struct {
    int32_t T, d, l, N, K, m;
    int32_t dtype;    /* 0: float32 arrays, 1: bfloat16 bit patterns */
    int32_t standard; /* 1: no projections (requires l == d) */
    int32_t m_shared; /* width of the shared expert, 0: none */
    int32_t expert_format; /* 0: the layer's dtype, 1: E4M3 + row scales, 2: MXFP4 */
    int32_t n_zero, n_copy, n_const; /* zero-computation experts (ids N ...) */
} oracle_dims;

/* routed ids: the FFN experts and the zero-computation experts */
static int routed_ids(const oracle_dims* D) { return D->N + D->n_zero + D->n_copy + D->n_const; }

static double widen(const void* base, int dtype, size_t i) {
    if (dtype == 0) return (double)((const float*)base)[i];
    uint32_t bits = ((uint32_t)((const uint16_t*)base)[i]) << 16;
    float f;
    memcpy(&f, &bits, sizeof f);
    return (double)f;
}

/* OCP FP8 E4M3 ("fn"): the value of one code */
static double e4m3(uint8_t c) {
    const int sign = c >> 7, ex = (c >> 3) & 15, man = c & 7;
    double v;
    if (ex == 15 && man == 7)
        v = NAN;
    else if (ex == 0)
        v = ldexp((double)man, -9); /* subnormal: (man / 8) * 2^-6 */
    else
        v = ldexp(1.0 + man / 8.0, ex - 7);
    return sign ? -v : v;
}

/* OCP MX E2M1 (FP4): the value of one 4-bit code */
static double e2m1(int c) {
    const int ex = (c >> 1) & 3, man = c & 1;
    const double v = ex == 0 ? 0.5 * man : ldexp(1.0 + 0.5 * man, ex - 1);
    return (c & 8) ? -v : v;
}

/* OCP MX E8M0 block scale: 2^(b - 127); 0xFF is NaN */
static double e8m0(uint8_t b) { return b == 0xFF ? NAN : ldexp(1.0, (int)b - 127); }

/* element i of a flattened expert weight matrix (row `row` holds it) */
static double expert_w(const oracle_dims* D, const void* W, const void* scale, size_t i, size_t row) {
    if (D->expert_format == 1) return e4m3(((const uint8_t*)W)[i]) * (double)((const float*)scale)[row];
    if (D->expert_format == 2) {
        const uint8_t byte = ((const uint8_t*)W)[i >> 1];
        return e2m1((i & 1) ? byte >> 4 : byte & 15) * e8m0(((const uint8_t*)scale)[i >> 5]);
    }
    return widen(W, D->dtype, i);
}

/*
 * Step 8: zero-computation expert q (counted from id N: zero experts, then
 * copy, then constant) with gate g adds g * y to s.
 */
static void zero_computation_expert(const oracle_dims* D, int q, const double* z, const void* zc,
                                    double g, double* s) {
    if (q < D->n_zero) return; /* zero expert: y = 0 */
    q -= D->n_zero;
    if (q < D->n_copy) { /* copy expert: y = z */
        for (int i = 0; i < D->l; ++i) s[i] += g * z[i];
        return;
    }
    q -= D->n_copy; /* constant expert q: y = c_q */
    for (int i = 0; i < D->l; ++i) s[i] += g * widen(zc, D->dtype, (size_t)q * D->l + i);
}

/* logit order: a outranks b if its logit is larger, or equal with a lower index */
static int outranks(const double* logit, int a, int b) {
    return logit[a] > logit[b] || (logit[a] == logit[b] && a < b);
}

/*
 * One token.  `forced` (K ids or NULL) replaces the token's own selection:
 * used when a caller wants this token evaluated with another routing (the
 * gates still come from this token's own fp64 logits).
 */
static void one_token(const oracle_dims* D, int t, const void* x, const void* Wd,
                      const void* Wr, const void* W1, const void* W2, const void* Wu,
                      const void* Ws1, const void* Ws2, const void* s1, const void* s2,
                      const void* zc, const float* bias, const int32_t* forced, double* out_t,
                      int32_t* ids_t, double* gates_t, double* logits_t, double* gap_t,
                      double* work) {
    const int d = D->d, l = D->l, N = D->N, K = D->K, m = D->m, dt = D->dtype;
    const int Nr = routed_ids(D);
    double* xt = work;            /* [d] */
    double* z = xt + d;           /* [l] */
    double* p = z + l;            /* [Nr] */
    double* h = p + Nr;           /* [m] */
    double* s = h + m;            /* [l] */
    double* hs = s + l;           /* [m_shared] */
    char* chosen = (char*)(hs + D->m_shared); /* [Nr] */

    for (int i = 0; i < d; ++i) xt[i] = widen(x, dt, (size_t)t * d + i);

    /* step 1: z = W_down x */
    if (D->standard) {
        for (int i = 0; i < l; ++i) z[i] = xt[i];
    } else {
        for (int j = 0; j < l; ++j) {
            double acc = 0.0;
            for (int i = 0; i < d; ++i) acc += widen(Wd, dt, (size_t)j * d + i) * xt[i];
            z[j] = acc;
        }
    }

    /* step 2: router logits at full d, one per routed id */
    for (int e = 0; e < Nr; ++e) {
        double acc = 0.0;
        for (int i = 0; i < d; ++i) acc += widen(Wr, dt, (size_t)e * d + i) * xt[i];
        if (bias) acc += (double)bias[e];
        logits_t[e] = acc;
    }

    /* step 3a: softmax over all Nr routed ids, max subtracted */
    double mx = logits_t[0];
    for (int e = 1; e < Nr; ++e) if (logits_t[e] > mx) mx = logits_t[e];
    double den = 0.0;
    for (int e = 0; e < Nr; ++e) { p[e] = exp(logits_t[e] - mx); den += p[e]; }
    for (int e = 0; e < Nr; ++e) p[e] /= den;

    /* step 3b: the K best ids in rank order (largest logit, then lowest index) */
    memset(chosen, 0, (size_t)Nr);
    for (int k = 0; k < K; ++k) {
        int best = -1;
        for (int e = 0; e < Nr; ++e)
            if (!chosen[e] && (best < 0 || outranks(logits_t, e, best))) best = e;
        chosen[best] = 1;
        ids_t[k] = best;
    }
    if (K < Nr) {
        int next = -1;
        for (int e = 0; e < Nr; ++e)
            if (!chosen[e] && (next < 0 || outranks(logits_t, e, next))) next = e;
        *gap_t = logits_t[ids_t[K - 1]] - logits_t[next];
    } else {
        *gap_t = INFINITY;
    }
    if (forced) for (int k = 0; k < K; ++k) ids_t[k] = forced[k];

    /* step 3c: renormalise the kept probabilities */
    double kept = 0.0;
    for (int k = 0; k < K; ++k) kept += p[ids_t[k]];
    for (int k = 0; k < K; ++k) gates_t[k] = p[ids_t[k]] / kept;

    /* steps 4-5: experts in latent space, gate-weighted sum in rank order */
    for (int i = 0; i < l; ++i) s[i] = 0.0;
    for (int k = 0; k < K; ++k) {
        const size_t e = (size_t)ids_t[k];
        if (ids_t[k] >= N) {
            zero_computation_expert(D, ids_t[k] - N, z, zc, gates_t[k], s);
            continue;
        }
        for (int j = 0; j < m; ++j) {
            double acc = 0.0;
            for (int i = 0; i < l; ++i) acc += expert_w(D, W1, s1, (e * m + j) * l + i, e * m + j) * z[i];
            double a = acc > 0.0 ? acc : 0.0;
            h[j] = a * a;
        }
        for (int i = 0; i < l; ++i) {
            double acc = 0.0;
            for (int j = 0; j < m; ++j) acc += expert_w(D, W2, s2, (e * l + i) * m + j, e * l + i) * h[j];
            s[i] += gates_t[k] * acc;
        }
    }

    /* step 6: project back to d and add the residual */
    for (int n = 0; n < d; ++n) {
        double acc;
        if (D->standard) {
            acc = s[n];
        } else {
            acc = 0.0;
            for (int i = 0; i < l; ++i) acc += widen(Wu, dt, (size_t)n * l + i) * s[i];
        }
        out_t[n] = xt[n] + acc;
    }

    /* step 7: the shared expert at full d, added to the output */
    const int ms = D->m_shared;
    if (ms > 0) {
        for (int j = 0; j < ms; ++j) {
            double acc = 0.0;
            for (int i = 0; i < d; ++i) acc += widen(Ws1, dt, (size_t)j * d + i) * xt[i];
            const double r = acc < 0.0 ? 0.0 : acc;
            hs[j] = r * r;
        }
        for (int n = 0; n < d; ++n) {
            double acc = 0.0;
            for (int j = 0; j < ms; ++j) acc += widen(Ws2, dt, (size_t)n * ms + j) * hs[j];
            out_t[n] += acc;
        }
    }
}

/*
 * oracle_forward: evaluate `n_sel` tokens (token indices in `sel`, or the
 * first n_sel tokens when sel is NULL).  Outputs are indexed by position in
 * the selection:  out [n_sel,d]  ids [n_sel,K]  gates [n_sel,K]
 * logits [n_sel,Nr]  gap [n_sel]  (gap = K-th minus (K+1)-th largest logit).
 * forced_ids [n_sel,K] or NULL.  Ws1 / Ws2: the shared expert, used only
 * when D->m_shared > 0.  s1 / s2: the expert weights' scales (FP8: float32
 * [N*m] / [N*l]; MXFP4: bytes [N*m*l/32] / [N*l*m/32]), used only when
 * D->expert_format != 0.  zc [n_const*l]: the constant
 * experts' vectors, used only when D->n_const > 0.  Returns 0, or -1 on bad
 * arguments.
 */
int oracle_forward(const oracle_dims* D, const void* x, const void* Wd, const void* Wr,
                   const void* W1, const void* W2, const void* Wu, const void* Ws1,
                   const void* Ws2, const void* s1, const void* s2, const void* zc,
                   const float* bias, const int32_t* sel, int32_t n_sel, const int32_t* forced_ids,
                   double* out, int32_t* ids, double* gates, double* logits, double* gap) {
    if (!D || !x || !Wr || !W1 || !W2 || !out || !ids || !gates || !logits || !gap) return -1;
    if (D->n_zero < 0 || D->n_copy < 0 || D->n_const < 0 || (D->n_const > 0 && !zc)) return -1;
    if (D->K < 1 || D->K > routed_ids(D) || D->T < 0 || n_sel < 0 || D->m_shared < 0) return -1;
    if (D->standard ? (D->l != D->d) : (!Wd || !Wu)) return -1;
    if (D->m_shared > 0 && (!Ws1 || !Ws2)) return -1;
    if (D->expert_format < 0 || D->expert_format > 2 || (D->expert_format != 0 && (!s1 || !s2))) return -1;
    if (D->expert_format == 2 && (D->l % 32 != 0 || D->m % 32 != 0)) return -1;
    for (int q = 0; q < n_sel; ++q) {
        int t = sel ? sel[q] : q;
        if (t < 0 || t >= D->T) return -1;
    }
    const size_t work_doubles =
        (size_t)D->d + 2 * (size_t)D->l + routed_ids(D) + D->m + D->m_shared + (routed_ids(D) + 7) / 8 + 1;
    int bad = 0;
#pragma omp parallel
    {
        double* work = (double*)malloc(work_doubles * sizeof(double));
        if (!work) {
#pragma omp atomic write
            bad = 1;
        } else {
#pragma omp for schedule(dynamic, 1)
            for (int q = 0; q < n_sel; ++q) {
                int t = sel ? sel[q] : q;
                one_token(D, t, x, Wd, Wr, W1, W2, Wu, Ws1, Ws2, s1, s2, zc, bias,
                          forced_ids ? forced_ids + (size_t)q * D->K : NULL,
                          out + (size_t)q * D->d, ids + (size_t)q * D->K,
                          gates + (size_t)q * D->K, logits + (size_t)q * routed_ids(D), gap + q, work);
            }
            free(work);
        }
    }
    return bad ? -1 : 0;
}

#ifdef _OPENMP
#include <omp.h>
#endif

/* number of threads the next oracle_forward call will use */
int oracle_threads(void) {
#ifdef _OPENMP
    return omp_get_max_threads();
#else
    return 1;
#endif
}

void oracle_set_threads(int n) {
#ifdef _OPENMP
    if (n > 0) omp_set_num_threads(n);
#else
    (void)n;
#endif
}
