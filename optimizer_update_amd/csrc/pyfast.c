/* pyfast.c -- CPython entry points for the per-step calls of
 * liboptimizer_update.so.
 *
 * The same C functions the ctypes binding calls (optimizer_update_32bit,
 * optimizer_update_8bit_blockwise, ou_plan_step, ou_plan8_step), with the
 * same positional arguments, converted here instead of by ctypes: about
 * 0.34 us per call against ctypes' 1.89 us (measured on the host with the
 * library stopping after its argument checks), which is most of the host
 * cost of a small tensor's update from Python.  Argument marshalling only:
 * every check and every step of the update stays in the library.
 *
 * Conversions follow ctypes': integers with __index__, floats rounded once
 * to binary32 (as c_float does), pointers from an int, None (NULL) or an
 * object with an int `value` (c_void_p).  A struct argument (the ou_hparams
 * of a plan step) is None, an int address, or an object exporting a buffer
 * of exactly sizeof(ou_hparams) bytes (an ou_hparams ctypes Structure),
 * whose address is passed; any other object (a ctypes pointer, a
 * c_void_p, a short bytearray) raises TypeError instead of letting the
 * library read past it.
 *
 * The library calls run with the GIL released, as ctypes' calls do: a
 * launch can block while the device queue is full, and other Python
 * threads keep running meanwhile.
 */
#define PY_SSIZE_T_CLEAN
#include <Python.h>
#include <stdint.h>

#include "../../include/optimizer_update.h"

static int to_i64(PyObject* o, long long* out)
{
    *out = PyLong_AsLongLong(o);
    return !(*out == -1 && PyErr_Occurred());
}

static int to_i32(PyObject* o, int* out)
{
    long long v;
    if (!to_i64(o, &v)) return 0;
    *out = (int)v;
    return 1;
}

static int to_f32(PyObject* o, float* out)
{
    const double d = PyFloat_AsDouble(o);
    if (d == -1.0 && PyErr_Occurred()) return 0;
    *out = (float)d;
    return 1;
}

static int to_ptr(PyObject* o, void** out)
{
    if (o == Py_None) {
        *out = NULL;
        return 1;
    }
    if (PyLong_Check(o)) {
        const unsigned long long v = PyLong_AsUnsignedLongLong(o);
        if (v == (unsigned long long)-1 && PyErr_Occurred()) return 0;
        *out = (void*)(uintptr_t)v;
        return 1;
    }
    PyObject* v = PyObject_GetAttrString(o, "value");   /* c_void_p */
    if (!v) return 0;
    const int ok = to_ptr(v, out);
    Py_DECREF(v);
    return ok;
}

static int to_struct_ptr(PyObject* o, const void** out)
{
    if (o == Py_None || PyLong_Check(o)) return to_ptr(o, (void**)out);
    Py_buffer view;
    if (!PyObject_CheckBuffer(o) || PyObject_GetBuffer(o, &view, PyBUF_SIMPLE) != 0) {
        PyErr_Clear();
        PyErr_Format(PyExc_TypeError, "expected an ou_hparams structure, an int address or None, not %.100s",
                     Py_TYPE(o)->tp_name);
        return 0;
    }
    const Py_ssize_t len = view.len;
    *out = view.buf;      /* the caller's argument keeps the object alive */
    PyBuffer_Release(&view);
    if (len != (Py_ssize_t)sizeof(ou_hparams)) {
        PyErr_Format(PyExc_TypeError,
                     "expected an ou_hparams structure (%zd bytes), got a %zd-byte %.100s buffer",
                     (Py_ssize_t)sizeof(ou_hparams), len, Py_TYPE(o)->tp_name);
        return 0;
    }
    return 1;
}

static int nargs_ok(const char* name, Py_ssize_t got, Py_ssize_t want)
{
    if (got == want) return 1;
    PyErr_Format(PyExc_TypeError, "%s takes %zd arguments (%zd given)", name, want, got);
    return 0;
}

/* optimizer_update_32bit(kind, dtype, param, grad, state1, state2, n, beta1,
 * beta2, beta3, alpha, eps, weight_decay, step, lr, skip_zeros, stream) */
static PyObject* py_update32(PyObject* self, PyObject* const* a, Py_ssize_t na)
{
    (void)self;
    if (!nargs_ok("optimizer_update_32bit", na, 17)) return NULL;
    int kind, dtype, skip;
    void *p, *g, *s1, *s2, *stream;
    long long n, step;
    float b1, b2, b3, alpha, eps, wd, lr;
    if (!to_i32(a[0], &kind) || !to_i32(a[1], &dtype) || !to_ptr(a[2], &p) || !to_ptr(a[3], &g) ||
        !to_ptr(a[4], &s1) || !to_ptr(a[5], &s2) || !to_i64(a[6], &n) || !to_f32(a[7], &b1) ||
        !to_f32(a[8], &b2) || !to_f32(a[9], &b3) || !to_f32(a[10], &alpha) || !to_f32(a[11], &eps) ||
        !to_f32(a[12], &wd) || !to_i64(a[13], &step) || !to_f32(a[14], &lr) || !to_i32(a[15], &skip) ||
        !to_ptr(a[16], &stream))
        return NULL;
    int st;
    Py_BEGIN_ALLOW_THREADS
    st = optimizer_update_32bit(kind, dtype, p, g, (float*)s1, (float*)s2, (int64_t)n, b1, b2, b3, alpha, eps,
                                wd, (int64_t)step, lr, skip, stream);
    Py_END_ALLOW_THREADS
    return PyLong_FromLong(st);
}

/* optimizer_update_8bit_blockwise(kind, dtype, param, grad, state1, state2,
 * absmax1, absmax2, n, beta1, beta2, beta3, alpha, eps, weight_decay, step,
 * lr, skip_zeros, stream) */
static PyObject* py_update8(PyObject* self, PyObject* const* a, Py_ssize_t na)
{
    (void)self;
    if (!nargs_ok("optimizer_update_8bit_blockwise", na, 19)) return NULL;
    int kind, dtype, skip;
    void *p, *g, *c1, *c2, *a1, *a2, *stream;
    long long n, step;
    float b1, b2, b3, alpha, eps, wd, lr;
    if (!to_i32(a[0], &kind) || !to_i32(a[1], &dtype) || !to_ptr(a[2], &p) || !to_ptr(a[3], &g) ||
        !to_ptr(a[4], &c1) || !to_ptr(a[5], &c2) || !to_ptr(a[6], &a1) || !to_ptr(a[7], &a2) ||
        !to_i64(a[8], &n) || !to_f32(a[9], &b1) || !to_f32(a[10], &b2) || !to_f32(a[11], &b3) ||
        !to_f32(a[12], &alpha) || !to_f32(a[13], &eps) || !to_f32(a[14], &wd) || !to_i64(a[15], &step) ||
        !to_f32(a[16], &lr) || !to_i32(a[17], &skip) || !to_ptr(a[18], &stream))
        return NULL;
    int st;
    Py_BEGIN_ALLOW_THREADS
    st = optimizer_update_8bit_blockwise(kind, dtype, p, g, (uint8_t*)c1, (uint8_t*)c2, (float*)a1, (float*)a2,
                                         (int64_t)n, b1, b2, b3, alpha, eps, wd, (int64_t)step, lr, skip, stream);
    Py_END_ALLOW_THREADS
    return PyLong_FromLong(st);
}

/* ou_plan_step(plan, hparams, stream) */
static PyObject* py_plan_step(PyObject* self, PyObject* const* a, Py_ssize_t na)
{
    (void)self;
    if (!nargs_ok("ou_plan_step", na, 3)) return NULL;
    void *plan, *stream;
    const void* hp;
    if (!to_ptr(a[0], &plan) || !to_struct_ptr(a[1], &hp) || !to_ptr(a[2], &stream)) return NULL;
    int st;
    Py_BEGIN_ALLOW_THREADS
    st = ou_plan_step((ou_plan)plan, (const ou_hparams*)hp, stream);
    Py_END_ALLOW_THREADS
    return PyLong_FromLong(st);
}

/* ou_plan8_step(plan, hparams, stream) */
static PyObject* py_plan8_step(PyObject* self, PyObject* const* a, Py_ssize_t na)
{
    (void)self;
    if (!nargs_ok("ou_plan8_step", na, 3)) return NULL;
    void *plan, *stream;
    const void* hp;
    if (!to_ptr(a[0], &plan) || !to_struct_ptr(a[1], &hp) || !to_ptr(a[2], &stream)) return NULL;
    int st;
    Py_BEGIN_ALLOW_THREADS
    st = ou_plan8_step((ou_plan8)plan, (const ou_hparams*)hp, stream);
    Py_END_ALLOW_THREADS
    return PyLong_FromLong(st);
}

static PyMethodDef methods[] = {
    {"optimizer_update_32bit", (PyCFunction)(void (*)(void))py_update32, METH_FASTCALL, NULL},
    {"optimizer_update_8bit_blockwise", (PyCFunction)(void (*)(void))py_update8, METH_FASTCALL, NULL},
    {"ou_plan_step", (PyCFunction)(void (*)(void))py_plan_step, METH_FASTCALL, NULL},
    {"ou_plan8_step", (PyCFunction)(void (*)(void))py_plan8_step, METH_FASTCALL, NULL},
    {NULL, NULL, 0, NULL},
};

static struct PyModuleDef module = {PyModuleDef_HEAD_INIT, "_fast", NULL, -1, methods,
                                    NULL, NULL, NULL, NULL};

PyMODINIT_FUNC PyInit__fast(void) { return PyModule_Create(&module); }
