/*
 * oracle.c -- fp64 CPU oracle of the delta-rule forward pass.
 *
 * TEST INFRASTRUCTURE ONLY.  Nothing in the product library calls, links or
 * includes this file; only the tests, the smoke check and the benchmark's CPU
 * baseline leg load it.  It shares no source with the GPU path.
 *
 * What it computes is the definition of the recurrence, token by token, in fp64, with no
 * chunking, blocking or reordering.  For each (b, h) the d_k x d_v state starts at S0 (or 0);
 * token i multiplies the state by its gate g_i and then applies its n_h Householder steps in
 * order, H_{i,j} = (I - beta_{i,j} k_{i,j} k_{i,j}^T) H_{i,j-1} + beta_{i,j} k_{i,j} v_{i,j}^T
 * (each step computed as the rank-1 write of the residual v - H^T k, which is the same matrix);
 * its output is scale * H_{i,n_h}^T q_i; the state after the last token is S_final.
 *
 * Sources (cited by page title and section; the equations, not any listing):
 *  - "08 linear delta rule & DPLR" page, section 1.2: S_t = (I - beta k k^T) S_{t-1} + beta k v^T
 *    (equal to the erase-write form of section 1.1), read out as o_t = S_t^T q_t.
 *  - same page, section 3 (Gated DeltaNet): S_t = (I - beta k k^T) alpha_t S_{t-1} + beta k v^T
 *    with a scalar alpha_t, which commutes with the Householder factor.
 *  - DeltaProduct reading notes, section 2.2 (n_h Householder factors per token) and section 2.6
 *    (the gated form H_{i,0} = g_i H_{i-1}, A_i = g_i F_{i,n_h} ... F_{i,1}), section 4.1 (keys,
 *    values and betas of a token's sub-steps consecutive; one output per token after its last
 *    sub-step).
 *
 * The gate enters as log g (fp32), exponentiated here in fp64; log g = -inf is
 * an exact reset (g = 0).  Inputs are float32 arrays holding exactly the values
 * the GPU receives (bf16 values are exact in float32); all arithmetic is fp64.
 *
 * Layouts (row-major, contiguous):
 *   q [B, L, H, dk]      k [B, L*n_h, H, dk]   v [B, L*n_h, H, dv]
 *   beta [B, L*n_h, H]   g_log [B, L, H] or NULL (ungated)
 *   S0 [B, H, dk, dv] or NULL (zeros)
 *   O [B, L, H, dv] fp64 out;  S_final [B, H, dk, dv] fp64 out or NULL.
 *
 * Pins: tests/test_oracle_pins.py checks this function against closed forms
 * (Householder eigenvalues, exact write at beta = 1, the n_h = 2 mod-3 rotation,
 * identical/orthogonal keys, beta = 2 twice, swap permutations, norm bound),
 * brute-force materialised products, the chunked UT/WY form and the DPLR loop.
 */
#include <math.h>
#include <stdlib.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

/* Returns 0 on success, -1 on allocation failure or bad sizes. */
int oracle_fwd(int B, int L, int H, int dk, int dv, int nh, double scale,
               const float* q, const float* k, const float* v, const float* beta,
               const float* g_log, const float* S0, double* O, double* S_final,
               int nthreads) {
    if (B < 0 || L < 0 || H <= 0 || dk <= 0 || dv <= 0 || nh <= 0) return -1;
    const long Lx = (long)L * nh;
    int fail = 0;
#ifdef _OPENMP
    if (nthreads > 0) omp_set_num_threads(nthreads);
#pragma omp parallel for schedule(dynamic, 1) reduction(| : fail)
#endif
    for (int bh = 0; bh < B * H; ++bh) {
        const int b = bh / H, h = bh % H;
        double* S = (double*)malloc(sizeof(double) * (size_t)dk * dv);
        double* e = (double*)malloc(sizeof(double) * (size_t)dv);
        if (!S || !e) { free(S); free(e); fail |= 1; continue; }
        /* S <- S0 (or 0) */
        for (int r = 0; r < dk; ++r)
            for (int c = 0; c < dv; ++c)
                S[(size_t)r * dv + c] =
                    S0 ? (double)S0[(((size_t)b * H + h) * dk + r) * dv + c] : 0.0;
        for (long i = 0; i < L; ++i) {
            /* gate once per token, before its Householder steps */
            if (g_log) {
                const double g = exp((double)g_log[((size_t)b * L + i) * H + h]);
                for (size_t x = 0; x < (size_t)dk * dv; ++x) S[x] *= g;
            }
            for (int j = 0; j < nh; ++j) {
                const long t = i * nh + j;
                const float* kt = k + (((size_t)b * Lx + t) * H + h) * dk;
                const float* vt = v + (((size_t)b * Lx + t) * H + h) * dv;
                const double bt = (double)beta[((size_t)b * Lx + t) * H + h];
                /* e = v_t - S^T k_t */
                for (int c = 0; c < dv; ++c) e[c] = (double)vt[c];
                for (int r = 0; r < dk; ++r) {
                    const double kr = (double)kt[r];
                    const double* Sr = S + (size_t)r * dv;
                    for (int c = 0; c < dv; ++c) e[c] -= Sr[c] * kr;
                }
                /* S = S + beta_t k_t e^T */
                for (int r = 0; r < dk; ++r) {
                    const double a = bt * (double)kt[r];
                    double* Sr = S + (size_t)r * dv;
                    for (int c = 0; c < dv; ++c) Sr[c] += a * e[c];
                }
            }
            /* o_i = scale * S^T q_i */
            const float* qi = q + (((size_t)b * L + i) * H + h) * dk;
            double* oi = O + (((size_t)b * L + i) * H + h) * dv;
            for (int c = 0; c < dv; ++c) oi[c] = 0.0;
            for (int r = 0; r < dk; ++r) {
                const double qr = (double)qi[r];
                const double* Sr = S + (size_t)r * dv;
                for (int c = 0; c < dv; ++c) oi[c] += Sr[c] * qr;
            }
            for (int c = 0; c < dv; ++c) oi[c] *= scale;
        }
        if (S_final)
            memcpy(S_final + ((size_t)b * H + h) * (size_t)dk * dv, S, sizeof(double) * (size_t)dk * dv);
        free(S);
        free(e);
    }
    return fail ? -1 : 0;
}

/*
 * oracle_fwd_kda -- the KDA recurrence ("08 linear delta rule & DPLR" page, section 1.4 table
 * and section 5: S_t = (I - beta_t k_t k_t^T) Diag(alpha_t) S_{t-1} + beta_t k_t v_t^T with a
 * decay per key channel, the diagonal applied first, then the Householder write), in fp64:
 *
 *   S <- S0 (or 0)
 *   for each token i:
 *       S[r][:] <- alpha_i[r] * S[r][:]                 (row r of S is key channel r)
 *       e <- v_i - S^T k_i;   S <- S + beta_i k_i e^T
 *       o_i <- scale * S^T q_i
 *
 * a_log [B, L, H, dk] float32 holds log alpha (exponentiated here in fp64).  One sub-step per
 * token.  Other arguments and layouts as oracle_fwd (n_h = 1).  Returns 0, or -1.
 * Pins: tests/test_oracle_pins.py (the page's DPLR reduction of KDA; equal channels give the
 * scalar-gated oracle_fwd; a zero channel decay erases that row of the state).
 */
int oracle_fwd_kda(int B, int L, int H, int dk, int dv, double scale,
                   const float* q, const float* k, const float* v, const float* beta,
                   const float* a_log, const float* S0, double* O, double* S_final, int nthreads) {
    if (B < 0 || L < 0 || H <= 0 || dk <= 0 || dv <= 0 || !a_log) return -1;
    int fail = 0;
#ifdef _OPENMP
    if (nthreads > 0) omp_set_num_threads(nthreads);
#pragma omp parallel for schedule(dynamic, 1) reduction(| : fail)
#endif
    for (int bh = 0; bh < B * H; ++bh) {
        const int b = bh / H, h = bh % H;
        double* S = (double*)malloc(sizeof(double) * (size_t)dk * dv);
        double* e = (double*)malloc(sizeof(double) * (size_t)dv);
        if (!S || !e) { free(S); free(e); fail |= 1; continue; }
        for (size_t x = 0; x < (size_t)dk * dv; ++x) S[x] = S0 ? (double)S0[((size_t)b * H + h) * dk * dv + x] : 0.0;
        for (long i = 0; i < L; ++i) {
            const size_t row = ((size_t)b * L + i) * H + h;   /* token-head index */
            for (int r = 0; r < dk; ++r) {
                const double a = exp((double)a_log[row * dk + r]);
                for (int c = 0; c < dv; ++c) S[(size_t)r * dv + c] *= a;
            }
            const float* ki = k + row * dk;
            const float* vi = v + row * dv;
            const double bt = (double)beta[row];
            for (int c = 0; c < dv; ++c) e[c] = (double)vi[c];
            for (int r = 0; r < dk; ++r)
                for (int c = 0; c < dv; ++c) e[c] -= S[(size_t)r * dv + c] * (double)ki[r];
            for (int r = 0; r < dk; ++r)
                for (int c = 0; c < dv; ++c) S[(size_t)r * dv + c] += bt * (double)ki[r] * e[c];
            const float* qi = q + row * dk;
            double* oi = O + row * dv;
            for (int c = 0; c < dv; ++c) {
                double a = 0.0;
                for (int r = 0; r < dk; ++r) a += S[(size_t)r * dv + c] * (double)qi[r];
                oi[c] = scale * a;
            }
        }
        if (S_final) memcpy(S_final + ((size_t)b * H + h) * (size_t)dk * dv, S, sizeof(double) * (size_t)dk * dv);
        free(S);
        free(e);
    }
    return fail ? -1 : 0;
}

/*
 * oracle_bwd -- gradients of the forward pass above, by reverse-mode differentiation of the
 * same recurrence, in fp64, with every intermediate state stored (no chunking).
 *
 * The pages give no gradient formulas; these follow from the recurrence by the chain rule.
 * With G = dLoss/dS for the state after a step (starting from dS_final, or 0):
 *   read    o_i = scale S^T q_i:          dq_i = scale S do_i;   G += scale q_i do_i^T
 *   write   S_a = S_b + beta k e^T, e = v - S_b^T k, u = G^T k:
 *           dv_t = beta u;   dbeta_t = u . e;   dk_t = beta (G e - S_b u);   G <- G - beta k u^T
 *   gate    S_{i,0} = g_i S_{i-1}:        dlog g_i = <G, S_{i,0}>;   G <- g_i G
 *   dS0 = G after the first token.
 * Steps are undone in reverse order: tokens from the last, and within a token its sub-steps
 * from the last, then its gate.
 *
 * Inputs as oracle_fwd, plus dO [B, L, H, dv] (float32) and dS_final [B, H, dk, dv] (float32
 * or NULL = 0).  Outputs fp64: dq [B, L, H, dk], dk [B, L*n_h, H, dk], dv [B, L*n_h, H, dv],
 * dbeta [B, L*n_h, H], dg_log [B, L, H] (ignored when g_log is NULL; may be NULL then),
 * dS0 [B, H, dk, dv].  Returns 0, or -1 on allocation failure or bad sizes.
 *
 * Pins: tests/test_oracle_pins.py compares every output with central finite differences of
 * oracle_fwd and with the closed form of a one-token sequence.
 */
int oracle_bwd(int B, int L, int H, int dk, int dv, int nh, double scale,
               const float* q, const float* k, const float* v, const float* beta,
               const float* g_log, const float* S0, const float* dO, const float* dS_final,
               double* dq, double* dkx, double* dvx, double* dbeta, double* dg_log, double* dS0,
               int nthreads) {
    if (B < 0 || L < 0 || H <= 0 || dk <= 0 || dv <= 0 || nh <= 0) return -1;
    const long Lx = (long)L * nh;
    const size_t SS = (size_t)dk * dv;
    int fail = 0;
#ifdef _OPENMP
    if (nthreads > 0) omp_set_num_threads(nthreads);
#pragma omp parallel for schedule(dynamic, 1) reduction(| : fail)
#endif
    for (int bh = 0; bh < B * H; ++bh) {
        const int b = bh / H, h = bh % H;
        /* Sb[t]: state before sub-step t; So[i]: state after token i (read by o_i) */
        double* Sb = (double*)malloc(sizeof(double) * SS * (size_t)(Lx > 0 ? Lx : 1));
        double* So = (double*)malloc(sizeof(double) * SS * (size_t)(L > 0 ? L : 1));
        double* S = (double*)malloc(sizeof(double) * SS);
        double* G = (double*)malloc(sizeof(double) * SS);
        double* e = (double*)malloc(sizeof(double) * (size_t)dv);
        double* u = (double*)malloc(sizeof(double) * (size_t)dv);
        if (!Sb || !So || !S || !G || !e || !u) {
            free(Sb); free(So); free(S); free(G); free(e); free(u);
            fail |= 1;
            continue;
        }
        /* forward, keeping the states */
        for (size_t x = 0; x < SS; ++x) S[x] = S0 ? (double)S0[((size_t)b * H + h) * SS + x] : 0.0;
        for (long i = 0; i < L; ++i) {
            if (g_log) {
                const double g = exp((double)g_log[((size_t)b * L + i) * H + h]);
                for (size_t x = 0; x < SS; ++x) S[x] *= g;
            }
            for (int j = 0; j < nh; ++j) {
                const long t = i * nh + j;
                const float* kt = k + (((size_t)b * Lx + t) * H + h) * dk;
                const float* vt = v + (((size_t)b * Lx + t) * H + h) * dv;
                const double bt = (double)beta[((size_t)b * Lx + t) * H + h];
                memcpy(Sb + (size_t)t * SS, S, sizeof(double) * SS);
                for (int c = 0; c < dv; ++c) e[c] = (double)vt[c];
                for (int r = 0; r < dk; ++r)
                    for (int c = 0; c < dv; ++c) e[c] -= S[(size_t)r * dv + c] * (double)kt[r];
                for (int r = 0; r < dk; ++r)
                    for (int c = 0; c < dv; ++c) S[(size_t)r * dv + c] += bt * (double)kt[r] * e[c];
            }
            memcpy(So + (size_t)i * SS, S, sizeof(double) * SS);
        }
        /* backward */
        for (size_t x = 0; x < SS; ++x) G[x] = dS_final ? (double)dS_final[((size_t)b * H + h) * SS + x] : 0.0;
        for (long i = L - 1; i >= 0; --i) {
            const float* qi = q + (((size_t)b * L + i) * H + h) * dk;
            const float* doi = dO + (((size_t)b * L + i) * H + h) * dv;
            double* dqi = dq + (((size_t)b * L + i) * H + h) * dk;
            const double* Si = So + (size_t)i * SS;
            for (int r = 0; r < dk; ++r) {
                double a = 0.0;
                for (int c = 0; c < dv; ++c) a += Si[(size_t)r * dv + c] * (double)doi[c];
                dqi[r] = scale * a;
            }
            for (int r = 0; r < dk; ++r)
                for (int c = 0; c < dv; ++c) G[(size_t)r * dv + c] += scale * (double)qi[r] * (double)doi[c];
            for (int j = nh - 1; j >= 0; --j) {
                const long t = i * nh + j;
                const float* kt = k + (((size_t)b * Lx + t) * H + h) * dk;
                const float* vt = v + (((size_t)b * Lx + t) * H + h) * dv;
                const double bt = (double)beta[((size_t)b * Lx + t) * H + h];
                const double* St = Sb + (size_t)t * SS;
                double* dkt = dkx + (((size_t)b * Lx + t) * H + h) * dk;
                double* dvt = dvx + (((size_t)b * Lx + t) * H + h) * dv;
                for (int c = 0; c < dv; ++c) { e[c] = (double)vt[c]; u[c] = 0.0; }
                for (int r = 0; r < dk; ++r)
                    for (int c = 0; c < dv; ++c) {
                        e[c] -= St[(size_t)r * dv + c] * (double)kt[r];
                        u[c] += G[(size_t)r * dv + c] * (double)kt[r];
                    }
                double db = 0.0;
                for (int c = 0; c < dv; ++c) {
                    dvt[c] = bt * u[c];
                    db += u[c] * e[c];
                }
                dbeta[((size_t)b * Lx + t) * H + h] = db;
                for (int r = 0; r < dk; ++r) {
                    double a = 0.0;
                    for (int c = 0; c < dv; ++c) a += G[(size_t)r * dv + c] * e[c] - St[(size_t)r * dv + c] * u[c];
                    dkt[r] = bt * a;
                }
                for (int r = 0; r < dk; ++r)
                    for (int c = 0; c < dv; ++c) G[(size_t)r * dv + c] -= bt * (double)kt[r] * u[c];
            }
            if (g_log) {
                /* the state right after the gate is the state before the token's first sub-step */
                const double g = exp((double)g_log[((size_t)b * L + i) * H + h]);
                const double* S0i = Sb + (size_t)(i * nh) * SS;
                double a = 0.0;
                for (size_t x = 0; x < SS; ++x) a += G[x] * S0i[x];
                if (dg_log) dg_log[((size_t)b * L + i) * H + h] = a;
                for (size_t x = 0; x < SS; ++x) G[x] *= g;
            }
        }
        memcpy(dS0 + ((size_t)b * H + h) * SS, G, sizeof(double) * SS);
        free(Sb); free(So); free(S); free(G); free(e); free(u);
    }
    return fail ? -1 : 0;
}

/* Number of threads OpenMP would use (for reporting the CPU baseline). */
int oracle_max_threads(void) {
#ifdef _OPENMP
    return omp_get_max_threads();
#else
    return 1;
#endif
}
