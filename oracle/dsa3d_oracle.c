/*
 * dsa3d_oracle.c -- plain, slow CPU oracle for 3D Deformable Slide Attention.
 *
 * TEST INFRASTRUCTURE ONLY. Only the tests, the smoke check and the
 * benchmark's CPU-baseline leg may load this file's library. The GPU library
 * shares no code, header, table or helper with it.
 *
 * What is computed (all arithmetic in double unless stated):
 *
 *   3D-DSA extends deformable attention to the temporal axis
 *   [MegaSlide-DiT, §5.1 Rationale]: every token (t,h,w) of a video-token grid
 *   attends, per head, to P points of its k_t x k_h x k_w spatiotemporal
 *   neighbourhood [MegaSlide-DiT (gist.science, Dutch and French summaries),
 *   "3D Deformable Slide Attention", Mechanism], each moved by a learned offset
 *   (dt,dh,dw); keys and values are read at the moved points by trilinear
 *   interpolation, i.e. grid_sample in bilinear mode on 5-D tensors
 *   [MegaSlide-DiT, §5.3 Implementation considerations], with zero padding;
 *   there is no causal mask [same section]; and with every offset zero the
 *   operator is plain fixed-window local attention [MegaSlide-DiT, §9.1 Effect
 *   of local offsets]. The formula of §5.2 is missing from the page text, so
 *   the steps below are the plain reading of those statements:
 *
 *   1. Window point p = (i_t,i_h,i_w), row-major over the window (w fastest).
 *      Reference point ref = x + dil * (i - (k-1)/2) in integers (window
 *      centred on the query; odd window sizes only).
 *   2. pos = float(ref) + float(offset), one IEEE single-precision add per axis;
 *      x0 = floorf(pos); f = pos - x0 as a single-precision subtraction. It is
 *      exact except for -0.5 < pos < 0, where f lands in [0.5, 1] and is rounded
 *      (possibly to 1.0: then corner x0 gets weight 0 and x0+1 weight 1). A
 *      position that is NaN, infinite or |pos| >= 2^30 puts the whole sample
 *      outside.
 *   3. k_p = sum over the 8 corners c in x0 + {0,1}^3 of w_c * K[c], with
 *      w_c = prod over axes of (c_axis ? f : 1 - f); a corner outside the token
 *      grid reads zero (it is never clamped and never wraps). v_p likewise.
 *   4. s_p = scale * <q, k_p>;  a = softmax(s) over all P points (points that
 *      land outside the grid are kept with their partial or zero key);
 *      lse = log sum_p exp(s_p).
 *   5. o = sum_p a_p v_p.
 *   Backward, for a loss L with dL/do = dO:
 *   6. da_p = <dO, v_p>;  ds_p = a_p (da_p - sum_j a_j da_j).
 *   7. dq = scale * sum_p ds_p k_p.
 *   8. dK[c] += w_c * scale * ds_p * q ;  dV[c] += w_c * a_p * dO  (in-grid c).
 *   9. dL/d(offset_p, axis) = sum_c (dw_c/df_axis) * (<scale ds_p q, K[c]> +
 *      <a_p dO, V[c]>), with dw_c/df_axis = (c_axis ? +1 : -1) times the other
 *      two axes' factors, and df/d(offset) = 1 (derivative taken inside the
 *      cell [x0, x0+1], i.e. from the right at exact integers).
 *
 * Every function works on one (batch item, head) at a time: a list of query
 * tokens given by absolute grid coordinates, and a K/V "box" -- a
 * sub-volume [bt0, bt0+BT) x [bh0, bh0+BH) x [bw0, bw0+BW) of the token grid
 * holding that head's key and value rows. The whole grid is the plain case; a
 * smaller box lets a test check sampled outputs of a very large grid. A corner
 * that lies inside the grid but outside the box is an error (return -1), never
 * a silent zero.
 *
 * Build: gcc -O2 -ffp-contract=off -fno-fast-math -fPIC -shared (x86-64 SSE
 * arithmetic: single-precision adds round to nearest even).
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

typedef struct {
    int32_t T, H, W;          /* token grid of one batch item */
    int32_t d;                /* head dimension */
    int32_t kt, kh, kw;       /* window shape, each odd */
    int32_t dil_t, dil_h, dil_w;
    double scale;             /* logit scale, normally 1/sqrt(d) */
    int32_t bt0, bh0, bw0;    /* K/V box origin (absolute token coordinates) */
    int32_t BT, BH, BW;       /* K/V box extent */
} orc_problem;

#define ORC_OUTSIDE INT32_MIN
#define ORC_ERR_BOX (-1)
#define ORC_ERR_ARG (-2)
#define ORC_ERR_MEM (-3)

int orc_version(void) { return 1; }

static int orc_check(const orc_problem* pr) {
    if (!pr || pr->T < 1 || pr->H < 1 || pr->W < 1 || pr->d < 1) return ORC_ERR_ARG;
    if (pr->kt < 1 || pr->kh < 1 || pr->kw < 1) return ORC_ERR_ARG;
    if (pr->kt % 2 == 0 || pr->kh % 2 == 0 || pr->kw % 2 == 0) return ORC_ERR_ARG;
    if (pr->dil_t < 1 || pr->dil_h < 1 || pr->dil_w < 1) return ORC_ERR_ARG;
    if (pr->BT < 0 || pr->BH < 0 || pr->BW < 0) return ORC_ERR_ARG;
    return 0;
}

/* Step 1-2: sample position of window point p of the query at x = (t,h,w).
 * Returns 1 and fills base/frac, or 0 when the sample lies entirely outside
 * (non-finite or huge position); then base = ORC_OUTSIDE and frac = 0. */
static int sample_point(const orc_problem* pr, const int32_t x[3], int p,
                        const float dlt[3], int32_t base[3], float frac[3]) {
    const int k[3] = {pr->kt, pr->kh, pr->kw};
    const int dil[3] = {pr->dil_t, pr->dil_h, pr->dil_w};
    const int idx[3] = {p / (k[1] * k[2]), (p / k[2]) % k[1], p % k[2]};
    float pos[3];
    for (int a = 0; a < 3; ++a) {
        int32_t ref = x[a] + dil[a] * (idx[a] - (k[a] - 1) / 2);
        pos[a] = (float)ref + dlt[a];
        if (!(fabsf(pos[a]) < 1073741824.0f)) {
            for (int b = 0; b < 3; ++b) { base[b] = ORC_OUTSIDE; frac[b] = 0.0f; }
            return 0;
        }
    }
    for (int a = 0; a < 3; ++a) {
        float fl = floorf(pos[a]);
        base[a] = (int32_t)fl;
        frac[a] = pos[a] - fl;
    }
    return 1;
}

/* Step 3 helper: corner c (bit 2 = t, bit 1 = h, bit 0 = w) of a sample.
 * Returns the box row index (>= 0), -2 when the corner is outside the grid
 * (reads zero), or -1 when it is inside the grid but outside the box. Also
 * returns the corner's trilinear weight and its three partial derivatives. */
static long corner(const orc_problem* pr, const int32_t base[3], const float frac[3], int c,
                   double* w, double dw[3]) {
    const int ct = (c >> 2) & 1, ch = (c >> 1) & 1, cw = c & 1;
    const double ft = frac[0], fh = frac[1], fw = frac[2];
    const double at = ct ? ft : 1.0 - ft, ah = ch ? fh : 1.0 - fh, aw = cw ? fw : 1.0 - fw;
    const double st = ct ? 1.0 : -1.0, sh = ch ? 1.0 : -1.0, sw = cw ? 1.0 : -1.0;
    *w = at * ah * aw;
    dw[0] = st * ah * aw;
    dw[1] = at * sh * aw;
    dw[2] = at * ah * sw;
    const int64_t t = (int64_t)base[0] + ct, h = (int64_t)base[1] + ch, x = (int64_t)base[2] + cw;
    if (t < 0 || t >= pr->T || h < 0 || h >= pr->H || x < 0 || x >= pr->W) return -2;
    if (t < pr->bt0 || t >= (int64_t)pr->bt0 + pr->BT || h < pr->bh0 || h >= (int64_t)pr->bh0 + pr->BH ||
        x < pr->bw0 || x >= (int64_t)pr->bw0 + pr->BW)
        return -1;
    return ((long)(t - pr->bt0) * pr->BH + (h - pr->bh0)) * (long)pr->BW + (x - pr->bw0);
}

/* Steps 1-3 for every point of one query: interpolated key/value rows. */
static int sample_rows(const orc_problem* pr, const int32_t x[3], const float* off,
                       const double* K, const double* V, double* kp, double* vp) {
    const int P = pr->kt * pr->kh * pr->kw, d = pr->d;
    for (int p = 0; p < P; ++p) {
        double* kr = kp + (long)p * d;
        double* vr = vp + (long)p * d;
        for (int e = 0; e < d; ++e) { kr[e] = 0.0; vr[e] = 0.0; }
        int32_t base[3];
        float frac[3];
        if (!sample_point(pr, x, p, off + 3L * p, base, frac)) continue;
        for (int c = 0; c < 8; ++c) {
            double w, dw[3];
            long r = corner(pr, base, frac, c, &w, dw);
            if (r == -1) return ORC_ERR_BOX;
            if (r < 0) continue;
            const double* Kc = K + r * d;
            const double* Vc = V + r * d;
            for (int e = 0; e < d; ++e) {
                kr[e] += w * Kc[e];
                vr[e] += w * Vc[e];
            }
        }
    }
    return 0;
}

/* Step 4: logits, softmax weights and log-sum-exp of one query. */
static void attend(int P, int d, double scale, const double* q, const double* kp,
                   double* s, double* a, double* lse) {
    double m = -INFINITY;
    for (int p = 0; p < P; ++p) {
        double acc = 0.0;
        for (int e = 0; e < d; ++e) acc += q[e] * kp[(long)p * d + e];
        s[p] = scale * acc;
        if (s[p] > m) m = s[p];
    }
    double z = 0.0;
    for (int p = 0; p < P; ++p) z += exp(s[p] - m);
    for (int p = 0; p < P; ++p) a[p] = exp(s[p] - m) / z;
    *lse = m + log(z);
}

/* Per-query geometry of every window point: base corner and fraction.
 * base/frac: [nq, P, 3]. Outside samples get base = INT32_MIN, frac = 0. */
int orc_geometry(const orc_problem* pr, long nq, const int32_t* qpos, const float* off,
                 int32_t* base, float* frac) {
    if (orc_check(pr)) return ORC_ERR_ARG;
    const int P = pr->kt * pr->kh * pr->kw;
    for (long i = 0; i < nq; ++i)
        for (int p = 0; p < P; ++p)
            sample_point(pr, qpos + 3 * i, p, off + (i * P + p) * 3, base + (i * P + p) * 3,
                         frac + (i * P + p) * 3);
    return 0;
}

/* Forward of nq queries of one (batch item, head).
 * qpos [nq,3] absolute (t,h,w); q [nq,d]; off [nq,P,3] (single precision);
 * K, V [BT,BH,BW,d] (the box); out o [nq,d], lse [nq], attn [nq,P] or NULL. */
int orc_forward(const orc_problem* pr, long nq, const int32_t* qpos, const double* q,
                const float* off, const double* K, const double* V,
                double* o, double* lse, double* attn) {
    if (orc_check(pr)) return ORC_ERR_ARG;
    const int P = pr->kt * pr->kh * pr->kw, d = pr->d;
    double* kp = malloc(sizeof(double) * (size_t)P * d);
    double* vp = malloc(sizeof(double) * (size_t)P * d);
    double* s = malloc(sizeof(double) * P);
    double* a = malloc(sizeof(double) * P);
    int rc = (kp && vp && s && a) ? 0 : ORC_ERR_MEM;
    for (long i = 0; i < nq && rc == 0; ++i) {
        rc = sample_rows(pr, qpos + 3 * i, off + i * P * 3, K, V, kp, vp);
        if (rc) break;
        attend(P, d, pr->scale, q + i * d, kp, s, a, lse + i);
        /* Step 5 */
        for (int e = 0; e < d; ++e) {
            double acc = 0.0;
            for (int p = 0; p < P; ++p) acc += a[p] * vp[(long)p * d + e];
            o[i * d + e] = acc;
        }
        if (attn)
            for (int p = 0; p < P; ++p) attn[i * P + p] = a[p];
    }
    free(kp); free(vp); free(s); free(a);
    return rc;
}

/* Backward of nq queries of one (batch item, head), recomputing the forward.
 * dout [nq,d]. Outputs: dq [nq,d] and doff [nq,P,3] are written; dK and dV
 * [BT,BH,BW,d] are ACCUMULATED (+=) so that the caller may split the queries
 * of one head over several calls. dK and dV may both be NULL when only the
 * query-side gradients are wanted (then calls on the same box may run
 * concurrently). */
int orc_backward(const orc_problem* pr, long nq, const int32_t* qpos, const double* q,
                 const float* off, const double* K, const double* V, const double* dout,
                 double* dq, double* doff, double* dK, double* dV) {
    if (orc_check(pr)) return ORC_ERR_ARG;
    const int P = pr->kt * pr->kh * pr->kw, d = pr->d;
    double* kp = malloc(sizeof(double) * (size_t)P * d);
    double* vp = malloc(sizeof(double) * (size_t)P * d);
    double* s = malloc(sizeof(double) * P);
    double* a = malloc(sizeof(double) * P);
    double* da = malloc(sizeof(double) * P);
    double* gk = malloc(sizeof(double) * d);
    double* gv = malloc(sizeof(double) * d);
    int rc = (kp && vp && s && a && da && gk && gv) ? 0 : ORC_ERR_MEM;
    for (long i = 0; i < nq && rc == 0; ++i) {
        const int32_t* x = qpos + 3 * i;
        const double* qi = q + i * d;
        const double* gi = dout + i * d;
        const float* oi = off + i * P * 3;
        rc = sample_rows(pr, x, oi, K, V, kp, vp);
        if (rc) break;
        double lse;
        attend(P, d, pr->scale, qi, kp, s, a, &lse);
        /* Step 6 */
        double sum_ada = 0.0;
        for (int p = 0; p < P; ++p) {
            double acc = 0.0;
            for (int e = 0; e < d; ++e) acc += gi[e] * vp[(long)p * d + e];
            da[p] = acc;
            sum_ada += a[p] * acc;
        }
        /* Step 7 */
        for (int e = 0; e < d; ++e) {
            double acc = 0.0;
            for (int p = 0; p < P; ++p) acc += a[p] * (da[p] - sum_ada) * kp[(long)p * d + e];
            dq[i * d + e] = pr->scale * acc;
        }
        /* Steps 8-9 */
        for (int p = 0; p < P; ++p) {
            const double ds = a[p] * (da[p] - sum_ada);
            for (int e = 0; e < d; ++e) {
                gk[e] = pr->scale * ds * qi[e];
                gv[e] = a[p] * gi[e];
            }
            double* dop = doff + (i * P + p) * 3;
            dop[0] = dop[1] = dop[2] = 0.0;
            int32_t base[3];
            float frac[3];
            if (!sample_point(pr, x, p, oi + 3L * p, base, frac)) continue;
            for (int c = 0; c < 8; ++c) {
                double w, dw[3];
                long r = corner(pr, base, frac, c, &w, dw);
                if (r == -1) { rc = ORC_ERR_BOX; break; }
                if (r < 0) continue;
                const double* Kc = K + r * d;
                const double* Vc = V + r * d;
                double dot = 0.0;
                for (int e = 0; e < d; ++e) dot += gk[e] * Kc[e] + gv[e] * Vc[e];
                if (dK && dV)
                    for (int e = 0; e < d; ++e) {
                        dK[r * d + e] += w * gk[e];
                        dV[r * d + e] += w * gv[e];
                    }
                dop[0] += dw[0] * dot;
                dop[1] += dw[1] * dot;
                dop[2] += dw[2] * dot;
            }
            if (rc) break;
        }
    }
    free(kp); free(vp); free(s); free(a); free(da); free(gk); free(gv);
    return rc;
}

/* Hybrid attention: sparse global tokens combined with local 3D-DSA
 * [MegaSlide-DiT, §11 Limitations and Discussion, future work (i)]. The pages
 * only name the idea; the reading here is the plainest one: every query of a
 * (batch item, head) attends, in ONE softmax, to its P sampled points (steps
 * 1-3) and to G global tokens whose key and value rows GK[g], GV[g] are the
 * same for every query of that (batch item, head):
 *   rows j = 0..P-1: k_p, v_p;  rows j = P..P+G-1: GK[j-P], GV[j-P]
 *   s_j = scale * <q, row_j>;  a = softmax(s) over all P+G rows;  o = sum_j a_j v_j
 * Backward over the same rows: da_j = <dO, v_j>, ds_j = a_j (da_j - sum_i a_i da_i),
 * dq = scale * sum_j ds_j k_j; the local rows scatter into dK, dV and the offsets
 * as in steps 8-9; the global rows give dGK[g] += scale ds_g q, dGV[g] += a_g dO.
 * GK, GV [G,d]; dGK, dGV [G,d] accumulated (+=). */
int orc_forward_hybrid(const orc_problem* pr, long nq, const int32_t* qpos, const double* q,
                       const float* off, const double* K, const double* V, int G,
                       const double* GK, const double* GV, double* o, double* lse) {
    if (orc_check(pr) || G < 0) return ORC_ERR_ARG;
    const int P = pr->kt * pr->kh * pr->kw, d = pr->d, R = P + G;
    double* kp = malloc(sizeof(double) * (size_t)R * d);
    double* vp = malloc(sizeof(double) * (size_t)R * d);
    double* s = malloc(sizeof(double) * R);
    double* a = malloc(sizeof(double) * R);
    int rc = (kp && vp && s && a) ? 0 : ORC_ERR_MEM;
    for (long i = 0; i < nq && rc == 0; ++i) {
        rc = sample_rows(pr, qpos + 3 * i, off + i * P * 3, K, V, kp, vp);
        if (rc) break;
        for (long e = 0; e < (long)G * d; ++e) {
            kp[(long)P * d + e] = GK[e];
            vp[(long)P * d + e] = GV[e];
        }
        attend(R, d, pr->scale, q + i * d, kp, s, a, lse + i);
        for (int e = 0; e < d; ++e) {
            double acc = 0.0;
            for (int j = 0; j < R; ++j) acc += a[j] * vp[(long)j * d + e];
            o[i * d + e] = acc;
        }
    }
    free(kp); free(vp); free(s); free(a);
    return rc;
}

int orc_backward_hybrid(const orc_problem* pr, long nq, const int32_t* qpos, const double* q,
                        const float* off, const double* K, const double* V, int G,
                        const double* GK, const double* GV, const double* dout,
                        double* dq, double* doff, double* dK, double* dV, double* dGK, double* dGV) {
    if (orc_check(pr) || G < 0) return ORC_ERR_ARG;
    const int P = pr->kt * pr->kh * pr->kw, d = pr->d, R = P + G;
    double* kp = malloc(sizeof(double) * (size_t)R * d);
    double* vp = malloc(sizeof(double) * (size_t)R * d);
    double* s = malloc(sizeof(double) * R);
    double* a = malloc(sizeof(double) * R);
    double* da = malloc(sizeof(double) * R);
    double* gk = malloc(sizeof(double) * d);
    double* gv = malloc(sizeof(double) * d);
    int rc = (kp && vp && s && a && da && gk && gv) ? 0 : ORC_ERR_MEM;
    for (long i = 0; i < nq && rc == 0; ++i) {
        const int32_t* x = qpos + 3 * i;
        const double* qi = q + i * d;
        const double* gi = dout + i * d;
        const float* oi = off + i * P * 3;
        rc = sample_rows(pr, x, oi, K, V, kp, vp);
        if (rc) break;
        for (long e = 0; e < (long)G * d; ++e) {
            kp[(long)P * d + e] = GK[e];
            vp[(long)P * d + e] = GV[e];
        }
        double lse;
        attend(R, d, pr->scale, qi, kp, s, a, &lse);
        double sum_ada = 0.0;
        for (int j = 0; j < R; ++j) {
            double acc = 0.0;
            for (int e = 0; e < d; ++e) acc += gi[e] * vp[(long)j * d + e];
            da[j] = acc;
            sum_ada += a[j] * acc;
        }
        for (int e = 0; e < d; ++e) {
            double acc = 0.0;
            for (int j = 0; j < R; ++j) acc += a[j] * (da[j] - sum_ada) * kp[(long)j * d + e];
            dq[i * d + e] = pr->scale * acc;
        }
        /* the global rows */
        for (int g = 0; g < G; ++g) {
            const double ds = a[P + g] * (da[P + g] - sum_ada);
            for (int e = 0; e < d; ++e) {
                dGK[(long)g * d + e] += pr->scale * ds * qi[e];
                dGV[(long)g * d + e] += a[P + g] * gi[e];
            }
        }
        /* the local rows: dK, dV and the offsets */
        for (int p = 0; p < P; ++p) {
            const double ds = a[p] * (da[p] - sum_ada);
            for (int e = 0; e < d; ++e) {
                gk[e] = pr->scale * ds * qi[e];
                gv[e] = a[p] * gi[e];
            }
            double* dop = doff + (i * P + p) * 3;
            dop[0] = dop[1] = dop[2] = 0.0;
            int32_t base[3];
            float frac[3];
            if (!sample_point(pr, x, p, oi + 3L * p, base, frac)) continue;
            for (int c = 0; c < 8; ++c) {
                double w, dw[3];
                long r = corner(pr, base, frac, c, &w, dw);
                if (r == -1) { rc = ORC_ERR_BOX; break; }
                if (r < 0) continue;
                const double* Kc = K + r * d;
                const double* Vc = V + r * d;
                double dot = 0.0;
                for (int e = 0; e < d; ++e) dot += gk[e] * Kc[e] + gv[e] * Vc[e];
                if (dK && dV)
                    for (int e = 0; e < d; ++e) {
                        dK[r * d + e] += w * gk[e];
                        dV[r * d + e] += w * gv[e];
                    }
                dop[0] += dw[0] * dot;
                dop[1] += dw[1] * dot;
                dop[2] += dw[2] * dot;
            }
            if (rc) break;
        }
    }
    free(kp); free(vp); free(s); free(a); free(da); free(gk); free(gv);
    return rc;
}
