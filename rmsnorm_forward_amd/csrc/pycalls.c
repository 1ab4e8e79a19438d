/* pycalls.c -- CPython entry points for the C ABI's per-call functions
 * (ln_fwd, rms_fwd, add_rms_fwd, rms_fp8_fwd, add_rms_fp8_fwd, ln_bwd,
 * rms_bwd), with the arguments and results of include/mi355norm.h.
 *
 * Argument marshalling only: each call converts its Python arguments (device
 * addresses as ints, None or 0 meaning NULL; sizes; eps and scale; the dtype
 * code; a stream handle or None) and calls the library's entry point, with
 * the interpreter lock released, returning its status code.  The functions
 * are reached through addresses handed over by _bind() from the process's
 * one loaded copy of libmi355norm.so, so this module links nothing.  It
 * exists because a ctypes call spends about 1.9 us converting eleven
 * arguments, and these functions are called once per normalisation. */
#define PY_SSIZE_T_CLEAN
#include <Python.h>
#include <limits.h>
#include <stdint.h>

typedef int (*fwd_fn)(const void*, const void*, const void*, void*, float*, float*, int64_t, int64_t, float, int,
                      void*);
typedef int (*add_fn)(const void*, const void*, const void*, void*, void*, float*, int64_t, int64_t, float, int,
                      void*);
typedef int (*fp8_fn)(const void*, const void*, void*, float*, int64_t, int64_t, float, float, int, void*);
typedef int (*add_fp8_fn)(const void*, const void*, const void*, void*, void*, float*, int64_t, int64_t, float,
                          float, int, void*);
typedef int (*ln_bwd_fn)(const void*, const void*, const void*, const float*, const float*, void*, float*, float*,
                         int64_t, int64_t, int, void*);
typedef int (*rms_bwd_fn)(const void*, const void*, const void*, const float*, void*, float*, int64_t, int64_t,
                          int, void*);

static fwd_fn p_ln_fwd, p_rms_fwd;
static add_fn p_add_rms_fwd;
static fp8_fn p_rms_fp8_fwd;
static add_fp8_fn p_add_rms_fp8_fwd;
static ln_bwd_fn p_ln_bwd;
static rms_bwd_fn p_rms_bwd;

/* an address: None or 0 is NULL; otherwise any integer (by __index__) */
static int addr(PyObject* o, void** out) {
    if (o == Py_None) {
        *out = NULL;
        return 1;
    }
    PyObject* i = PyNumber_Index(o);
    if (!i) return 0;
    const unsigned long long v = PyLong_AsUnsignedLongLongMask(i);
    Py_DECREF(i);
    if (PyErr_Occurred()) return 0;
    *out = (void*)(uintptr_t)v;
    return 1;
}

static int i64(PyObject* o, int64_t* out) {
    PyObject* i = PyNumber_Index(o);
    if (!i) return 0;
    const long long v = PyLong_AsLongLong(i);
    Py_DECREF(i);
    if (v == -1 && PyErr_Occurred()) return 0;
    *out = (int64_t)v;
    return 1;
}

/* the dtype code: an int of the ABI (out of range raises, never wraps) */
static int code(PyObject* o, int* out) {
    int64_t v;
    if (!i64(o, &v)) return 0;
    if (v < INT_MIN || v > INT_MAX) {
        PyErr_SetString(PyExc_OverflowError, "dtype code out of the range of a C int");
        return 0;
    }
    *out = (int)v;
    return 1;
}

static int f32(PyObject* o, float* out) {
    const double v = PyFloat_AsDouble(o);
    if (v == -1.0 && PyErr_Occurred()) return 0;
    *out = (float)v;
    return 1;
}

static int nargs(const char* name, Py_ssize_t n, Py_ssize_t want) {
    if (n == want) return 1;
    PyErr_Format(PyExc_TypeError, "%s takes %zd arguments (%zd given)", name, want, n);
    return 0;
}

static int bound(const void* f, const char* name) {
    if (f) return 1;
    PyErr_Format(PyExc_RuntimeError, "%s: the library's entry points are not bound", name);
    return 0;
}

/* x, gamma, beta, y, mean, rstd, M, N, eps, dtype, stream */
static PyObject* call_fwd(fwd_fn f, const char* name, PyObject* const* a, Py_ssize_t n) {
    void* p[6];
    void* stream;
    int64_t M, N;
    int dt;
    float eps;
    if (!nargs(name, n, 11) || !bound((const void*)f, name)) return NULL;
    for (int k = 0; k < 6; ++k)
        if (!addr(a[k], &p[k])) return NULL;
    if (!i64(a[6], &M) || !i64(a[7], &N) || !f32(a[8], &eps) || !code(a[9], &dt) || !addr(a[10], &stream)) return NULL;
    int st;
    Py_BEGIN_ALLOW_THREADS
    st = f(p[0], p[1], p[2], p[3], (float*)p[4], (float*)p[5], M, N, eps, dt, stream);
    Py_END_ALLOW_THREADS
    return PyLong_FromLong(st);
}

static PyObject* m_ln_fwd(PyObject* s, PyObject* const* a, Py_ssize_t n) {
    (void)s;
    return call_fwd(p_ln_fwd, "ln_fwd", a, n);
}

static PyObject* m_rms_fwd(PyObject* s, PyObject* const* a, Py_ssize_t n) {
    (void)s;
    return call_fwd(p_rms_fwd, "rms_fwd", a, n);
}

/* x, residual, gamma, y, residual_out, rstd, M, N, eps, dtype, stream */
static PyObject* m_add_rms_fwd(PyObject* s, PyObject* const* a, Py_ssize_t n) {
    (void)s;
    void* p[6];
    void* stream;
    int64_t M, N;
    int dt;
    float eps;
    if (!nargs("add_rms_fwd", n, 11) || !bound((const void*)p_add_rms_fwd, "add_rms_fwd")) return NULL;
    for (int k = 0; k < 6; ++k)
        if (!addr(a[k], &p[k])) return NULL;
    if (!i64(a[6], &M) || !i64(a[7], &N) || !f32(a[8], &eps) || !code(a[9], &dt) || !addr(a[10], &stream)) return NULL;
    int st;
    Py_BEGIN_ALLOW_THREADS
    st = p_add_rms_fwd(p[0], p[1], p[2], p[3], p[4], (float*)p[5], M, N, eps, dt, stream);
    Py_END_ALLOW_THREADS
    return PyLong_FromLong(st);
}

/* x, gamma, y, rstd, M, N, eps, scale, dtype, stream */
static PyObject* m_rms_fp8_fwd(PyObject* s, PyObject* const* a, Py_ssize_t n) {
    (void)s;
    void* p[4];
    void* stream;
    int64_t M, N;
    int dt;
    float eps, scale;
    if (!nargs("rms_fp8_fwd", n, 10) || !bound((const void*)p_rms_fp8_fwd, "rms_fp8_fwd")) return NULL;
    for (int k = 0; k < 4; ++k)
        if (!addr(a[k], &p[k])) return NULL;
    if (!i64(a[4], &M) || !i64(a[5], &N) || !f32(a[6], &eps) || !f32(a[7], &scale) || !code(a[8], &dt) ||
        !addr(a[9], &stream))
        return NULL;
    int st;
    Py_BEGIN_ALLOW_THREADS
    st = p_rms_fp8_fwd(p[0], p[1], p[2], (float*)p[3], M, N, eps, scale, dt, stream);
    Py_END_ALLOW_THREADS
    return PyLong_FromLong(st);
}

/* x, residual, gamma, y, residual_out, rstd, M, N, eps, scale, dtype, stream */
static PyObject* m_add_rms_fp8_fwd(PyObject* s, PyObject* const* a, Py_ssize_t n) {
    (void)s;
    void* p[6];
    void* stream;
    int64_t M, N;
    int dt;
    float eps, scale;
    if (!nargs("add_rms_fp8_fwd", n, 12) || !bound((const void*)p_add_rms_fp8_fwd, "add_rms_fp8_fwd")) return NULL;
    for (int k = 0; k < 6; ++k)
        if (!addr(a[k], &p[k])) return NULL;
    if (!i64(a[6], &M) || !i64(a[7], &N) || !f32(a[8], &eps) || !f32(a[9], &scale) || !code(a[10], &dt) ||
        !addr(a[11], &stream))
        return NULL;
    int st;
    Py_BEGIN_ALLOW_THREADS
    st = p_add_rms_fp8_fwd(p[0], p[1], p[2], p[3], p[4], (float*)p[5], M, N, eps, scale, dt, stream);
    Py_END_ALLOW_THREADS
    return PyLong_FromLong(st);
}

/* dy, x, gamma, mean, rstd, dx, dgamma, dbeta, M, N, dtype, stream */
static PyObject* m_ln_bwd(PyObject* s, PyObject* const* a, Py_ssize_t n) {
    (void)s;
    void* p[8];
    void* stream;
    int64_t M, N;
    int dt;
    if (!nargs("ln_bwd", n, 12) || !bound((const void*)p_ln_bwd, "ln_bwd")) return NULL;
    for (int k = 0; k < 8; ++k)
        if (!addr(a[k], &p[k])) return NULL;
    if (!i64(a[8], &M) || !i64(a[9], &N) || !code(a[10], &dt) || !addr(a[11], &stream)) return NULL;
    int st;
    Py_BEGIN_ALLOW_THREADS
    st = p_ln_bwd(p[0], p[1], p[2], (const float*)p[3], (const float*)p[4], p[5], (float*)p[6], (float*)p[7], M, N,
                  dt, stream);
    Py_END_ALLOW_THREADS
    return PyLong_FromLong(st);
}

/* dy, x, gamma, rstd, dx, dgamma, M, N, dtype, stream */
static PyObject* m_rms_bwd(PyObject* s, PyObject* const* a, Py_ssize_t n) {
    (void)s;
    void* p[6];
    void* stream;
    int64_t M, N;
    int dt;
    if (!nargs("rms_bwd", n, 10) || !bound((const void*)p_rms_bwd, "rms_bwd")) return NULL;
    for (int k = 0; k < 6; ++k)
        if (!addr(a[k], &p[k])) return NULL;
    if (!i64(a[6], &M) || !i64(a[7], &N) || !code(a[8], &dt) || !addr(a[9], &stream)) return NULL;
    int st;
    Py_BEGIN_ALLOW_THREADS
    st = p_rms_bwd(p[0], p[1], p[2], (const float*)p[3], p[4], (float*)p[5], M, N, dt, stream);
    Py_END_ALLOW_THREADS
    return PyLong_FromLong(st);
}

/* _bind(ln_fwd, rms_fwd, add_rms_fwd, rms_fp8_fwd, add_rms_fp8_fwd, ln_bwd,
 * rms_bwd): the entry points' addresses in the loaded library */
static PyObject* m_bind(PyObject* s, PyObject* const* a, Py_ssize_t n) {
    (void)s;
    void* p[7];
    if (!nargs("_bind", n, 7)) return NULL;
    for (int k = 0; k < 7; ++k) {
        if (!addr(a[k], &p[k])) return NULL;
        if (!p[k]) {
            PyErr_SetString(PyExc_ValueError, "_bind: a null entry point");
            return NULL;
        }
    }
    p_ln_fwd = (fwd_fn)p[0];
    p_rms_fwd = (fwd_fn)p[1];
    p_add_rms_fwd = (add_fn)p[2];
    p_rms_fp8_fwd = (fp8_fn)p[3];
    p_add_rms_fp8_fwd = (add_fp8_fn)p[4];
    p_ln_bwd = (ln_bwd_fn)p[5];
    p_rms_bwd = (rms_bwd_fn)p[6];
    Py_RETURN_NONE;
}

#define FAST(name, fn, doc) {name, (PyCFunction)(void (*)(void))fn, METH_FASTCALL, doc}
static PyMethodDef methods[] = {
    FAST("ln_fwd", m_ln_fwd, "LayerNorm forward on device addresses; returns the norm_status code."),
    FAST("rms_fwd", m_rms_fwd, "RMSNorm forward on device addresses; returns the norm_status code."),
    FAST("add_rms_fwd", m_add_rms_fwd, "Residual add then RMSNorm on device addresses; returns the norm_status code."),
    FAST("rms_fp8_fwd", m_rms_fp8_fwd, "RMSNorm with FP8 (E4M3) output on device addresses; returns the status."),
    FAST("add_rms_fp8_fwd", m_add_rms_fp8_fwd, "Residual add + RMSNorm with FP8 (E4M3) output on device addresses."),
    FAST("ln_bwd", m_ln_bwd,
         "LayerNorm backward on device addresses (dgamma / dbeta fp32 [N] or None); returns the norm_status code."),
    FAST("rms_bwd", m_rms_bwd, "RMSNorm backward on device addresses; returns the norm_status code."),
    FAST("_bind", m_bind, "Bind the library's entry points (their addresses)."),
    {NULL, NULL, 0, NULL}};

static struct PyModuleDef module = {PyModuleDef_HEAD_INIT, "_calls",
                                    "CPython entry points for libmi355norm.so's per-call functions.", -1, methods,
                                    NULL, NULL, NULL, NULL};

PyMODINIT_FUNC PyInit__calls(void) { return PyModule_Create(&module); }
